"""GPU parity of the Chebyshev solve with two-piece binary16 products (DASH_FP32_SPLIT16): each
product's operands are brought near 8 by a power of two per block and cut into two binary16 pieces
(22 of fp32's 24 significant bits), and three piece products accumulate in fp32.  The gates are
the fp32 ones (iterate parity 1e-4 against the oracle's fp64 Clenshaw recurrence, residual 1e-3),
and the solve must be as accurate as the one on the fp32 matrix cores (error within 1.5 times
theirs): the pieces' rounding (2^-22 of an element) is below the error the fp32 accumulation of a
product already makes.  Where the split does not apply (degree 2, B not a multiple of 256) the
result is the fp32 path's, bit for bit."""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import (DEV, ITERATE_TOL, R_FP32, frob_scale, host_frob_scale, host_power_scale, rel_err, residual,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu

S16 = dash.DASH_FP32_SPLIT16


def cheb_p(A, s, degree, lo, hi, prec):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, prec, device=DEV)
    dash.dash_inverse_root_cheb_prec(A, s, N, B, degree, lo, hi, prec, X, status=status, ws=ws)
    return X, status


def spectrum_stack(seed, N, B, lam_min=0.05):
    A = di.known_spectrum_stack(seed, N, B, lam_min, 1.0)[0].astype(np.float32)
    return A, to_dev(A)


def as_accurate_as_fp32(Ad, s, d, lo, hi, ref, err):
    Xf, _ = cheb_p(Ad, s, d, lo, hi, dash.DASH_FP32)
    err_f = rel_err(to_host(Xf), ref)
    print("fp32 err", err_f.max())
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)


@pytest.mark.parametrize("B,N,degrees", [(256, 4, (3, 4, 8, 24)), (512, 2, (24,)), (768, 2, (5, 24)),
                                         (1024, 1, (24,))])
def test_cheb_split16_matches_oracle(B, N, degrees):
    """Several 256-wide tiles per block, power-iteration scale, hi = 1.25; degree 3 (two products:
    the first and the last), 4 (three: every magnitude slot used once), 8 and 24 (the slots
    rotate).  B = 768: an odd number of tiles per side (6 upper-triangle tiles, 3 diagonal ones
    whose waves take the balanced regions, 48 k-slices)."""
    A, Ad = spectrum_stack(460 + B, N, B)
    s = host_power_scale(A, di.start_vectors(B, 32))
    lo, hi = 0.04, 1.25
    for d in degrees:
        X, status = cheb_p(Ad, s, d, lo, hi, S16)
        Xh = to_host(X)
        ref = oracle.cheb_inverse_root(A, to_host(s), d, lo, hi)
        err = rel_err(Xh, ref)
        print("B", B, "degree", d, "split16 err", err.max())
        assert np.all(to_host(status) == 0)
        assert err.max() < ITERATE_TOL
        assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))  # triangle-only products, mirrored
        if d == 24:
            assert residual(Xh, A).max() < R_FP32
            as_accurate_as_fp32(Ad, s, d, lo, hi, ref, err)


def test_cheb_split16_wide_magnitudes():
    """Blocks D A D with D log-uniform over six decades (elements from 1e-12 to 1 of one another,
    an interval reaching down to 1e-7): the small elements' pieces stay in binary16's normal range
    after the block's power of two, so the solve keeps the fp32 path's accuracy."""
    B, N = 256, 2
    g = di.rng(471)
    A64 = di.known_spectrum_stack(470, N, B, 0.05, 1.0)[0]
    D = np.exp(g.uniform(np.log(1e-3), 0.0, (N, B)))
    A = (D[:, :, None] * A64 * D[:, None, :]).astype(np.float32)
    A = (A + np.swapaxes(A, 1, 2)) / 2  # exactly symmetric
    Ad = to_dev(A)
    lam = np.linalg.eigvalsh(A.astype(np.float64))
    s = to_dev(lam[:, -1] * 1.01)
    lo = float(max(1e-7, 0.9 * (lam[:, 0] / (lam[:, -1] * 1.01)).min()))
    X, status = cheb_p(Ad, s, 24, lo, 1.25, S16)
    ref = oracle.cheb_inverse_root(A, to_host(s), 24, lo, 1.25)
    err = rel_err(to_host(X), ref)
    print("lo", lo, "split16 err", err.max())
    assert np.all(to_host(status) == 0)
    as_accurate_as_fp32(Ad, s, 24, lo, 1.25, ref, err)


def test_cheb_split16_falls_back_to_fp32_bitwise():
    """Degree 2 runs one product on the fp32 cores; B = 320 has no 256-wide tiling: both equal the
    fp32 path bit for bit."""
    A, Ad = spectrum_stack(472, 2, 256)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 2, 0.02, 1.0, S16)
    X2, _ = cheb_p(Ad, s, 2, 0.02, 1.0, dash.DASH_FP32)
    assert torch.equal(X1, X2)
    A, Ad = spectrum_stack(473, 2, 320)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 12, 0.02, 1.0, S16)
    X2, _ = cheb_p(Ad, s, 12, 0.02, 1.0, dash.DASH_FP32)
    assert torch.equal(X1, X2)


@pytest.mark.parametrize("e", [4, -40, 40])
def test_cheb_split16_scale_equivariance_and_batch_independence(e):
    """A power-of-two scale 2^e of A and s moves each block's power of two by -e and leaves every
    piece as it was, so X(2^e A, 2^e s) = 2^(-e/4) X(A, s) bit for bit; a permuted stack gives the
    permuted result, and one block alone its result in the stack (each block's bounds are its own)."""
    A, Ad = spectrum_stack(474, 4, 256)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 12, 0.02, 1.0, S16)
    Xe, _ = cheb_p(Ad * 2.0 ** e, s * 2.0 ** e, 12, 0.02, 1.0, S16)
    assert torch.equal(Xe * 2.0 ** (e / 4), X1)
    perm = torch.tensor([2, 0, 3, 1], device=DEV)
    Xp, _ = cheb_p(Ad[perm].contiguous(), s[perm].contiguous(), 12, 0.02, 1.0, S16)
    assert torch.equal(Xp, X1[perm])
    Xi, _ = cheb_p(Ad[2:3].contiguous(), s[2:3].contiguous(), 12, 0.02, 1.0, S16)
    assert torch.equal(Xi[0], X1[2])


def test_cheb_split16_flags_bad_blocks():
    """A zero or NaN scale flags bit 0 and gives a NaN block; a non-finite input element flags bit
    1; the other blocks are untouched (their magnitude bounds are their own)."""
    A, Ad = spectrum_stack(475, 4, 256)
    s = frob_scale(Ad).clone()
    X_good, st_good = cheb_p(Ad, s, 8, 0.02, 1.0, S16)
    assert np.all(to_host(st_good) == 0)
    s_bad = s.clone()
    s_bad[1] = 0.0
    s_bad[2] = float("nan")
    X, st = cheb_p(Ad, s_bad, 8, 0.02, 1.0, S16)
    assert np.array_equal(to_host(st).astype(int) & 1, [0, 1, 1, 0])
    assert np.all(np.isnan(to_host(X)[[1, 2]]))
    assert torch.equal(X[[0, 3]], X_good[[0, 3]])
    bad = Ad.clone()
    bad[0, 3, 5] = float("inf")
    bad[0, 5, 3] = float("inf")
    Xb, stb = cheb_p(bad, s, 8, 0.02, 1.0, S16)
    assert np.array_equal(to_host(stb).astype(int) & 2, [2, 0, 0, 0])
    assert torch.equal(Xb[1:], X_good[1:])


def test_cheb_split16_per_block_interval_matches_oracle():
    """dash_inverse_root_cheb_blocks with two-piece products: each block on its own interval
    [floor / s_i, 1.25], against the oracle on the same intervals."""
    B, N = 256, 3
    A, Ad = spectrum_stack(476, N, B, lam_min=0.01)
    A[1] *= 8.0
    A[2] *= 0.25
    Ad = to_dev(A)
    s = host_power_scale(A, di.start_vectors(B, 32))
    floor = 0.005
    X = torch.empty_like(Ad)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    lo_out = torch.empty(N, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, S16, device=DEV)
    dash.dash_inverse_root_cheb_blocks(Ad, s, N, B, 24, floor, None, 1.0, 1.25, S16, X, lo_out=lo_out,
                                       status=status, ws=ws)
    lo = oracle.cheb_interval_lo(to_host(s), floor)
    assert np.allclose(to_host(lo_out), lo, rtol=1e-6)
    ref = oracle.cheb_inverse_root(A, to_host(s), 24, lo, 1.25)
    err = rel_err(to_host(X), ref)
    print("per-block split16 err", err)
    assert np.all(to_host(status) == 0)
    assert err.max() < ITERATE_TOL


# ------------------------------------------------------------------------------------------------
# NDB with two-piece binary16 products (every product a general one, the right operand gathered by
# columns; each operand's bound from the launch that wrote it, or a pass over it)
# ------------------------------------------------------------------------------------------------

def ndb_p(A, s, it1, it2, prec, want_sqrt=False, want_monitor=False):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    R = torch.empty_like(A) if want_sqrt else None
    mon = torch.empty((N, it1 + it2), device=DEV) if want_monitor else None
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, prec, device=DEV)
    dash.dash_inverse_root_ndb_prec(A, s, N, B, it1, it2, prec, X, sqrt_out=R, monitor=mon, status=status, ws=ws)
    return X, R, mon, status


@pytest.fixture(scope="module")
def conditioned():
    A, _, _ = di.conditioned_stack()  # N = 16, B = 256, kappa = 1e4
    return A, to_dev(A)


@pytest.mark.parametrize("scaling", ["power", "frobenius"])
def test_ndb_split16_conditioned(conditioned, scaling):
    """kappa 1e4: the stability case of the non-symmetrised NDB iteration, at the fp32 gates, and as
    accurate as the fp32 matrix cores."""
    A, Ad = conditioned
    s = host_power_scale(A, di.start_vectors(256, 32)) if scaling == "power" else host_frob_scale(A)
    T = 16 if scaling == "power" else 18
    X, _, _, status = ndb_p(Ad, s, T, T, S16)
    X_ref, _, _ = oracle.ndb_inverse_root(A, to_host(s), T, T)
    err = rel_err(to_host(X), X_ref)
    Xf, _, _, _ = ndb_p(Ad, s, T, T, dash.DASH_FP32)
    err_f = rel_err(to_host(Xf), X_ref)
    print(scaling, "split16 err", err.max(), "fp32 err", err_f.max())
    assert err.max() < ITERATE_TOL
    assert residual(to_host(X), A).max() < R_FP32
    assert np.all(to_host(status) == 0)
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)


@pytest.mark.parametrize("it1,it2,B", [(1, 1, 512), (2, 3, 512), (4, 4, 512), (3, 3, 768)])
def test_ndb_split16_iterates_sqrt_and_monitor(it1, it2, B):
    """Several 256-wide tiles per block (B = 512, all 16 tiles; B = 768, 9): X, the square root and
    the monitor of every step against the oracle's NDB iterates (one step: the first product alone;
    two or more: the bounds handed from launch to launch)."""
    A, Ad = spectrum_stack(480, 2, B)
    s = host_frob_scale(A)
    X, R, mon, status = ndb_p(Ad, s, it1, it2, S16, want_sqrt=True, want_monitor=True)
    X_ref, R_ref, mon_ref = oracle.ndb_inverse_root(A, to_host(s), it1, it2, want_sqrt=True)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(rel_err(to_host(R), R_ref)) < ITERATE_TOL
    assert np.max(np.abs(to_host(mon) - mon_ref) / mon_ref) < 1e-3
    assert np.all(to_host(status) == 0)


def test_ndb_split16_fallback_equivariance_independence_and_flags(conditioned):
    """B = 320 has no 256-wide tiling: the fp32 path bit for bit.  At B = 256: X(16 A, 16 s) = X / 2
    bit for bit (every bound moves by the same power of two), one block alone equals its result in
    the stack, a bad scale flags bit 0 and leaves the other blocks untouched."""
    A, Ad = spectrum_stack(481, 2, 320)
    s = frob_scale(Ad)
    X1, _, _, _ = ndb_p(Ad, s, 5, 5, S16)
    X2, _, _, _ = ndb_p(Ad, s, 5, 5, dash.DASH_FP32)
    assert torch.equal(X1, X2)
    _, Ad = conditioned
    Ad = Ad[:4].contiguous()
    s = frob_scale(Ad)
    X, _, _, _ = ndb_p(Ad, s, 8, 8, S16)
    X16, _, _, _ = ndb_p(16 * Ad, 16 * s, 8, 8, S16)
    assert torch.equal(X16 * 2, X)
    Xi, _, _, _ = ndb_p(Ad[3:4].contiguous(), s[3:4].contiguous(), 8, 8, S16)
    assert torch.equal(Xi[0], X[3])
    s_bad = s.clone()
    s_bad[1] = float("nan")
    Xb, _, _, st = ndb_p(Ad, s_bad, 8, 8, S16)
    assert np.array_equal(to_host(st).astype(int) & 1, [0, 1, 0, 0])
    assert np.all(np.isnan(to_host(Xb)[1]))
    assert torch.equal(Xb[[0, 2, 3]], X[[0, 2, 3]])


# ------------------------------------------------------------------------------------------------
# The preconditioned update U = (XL G) XR with two-piece binary16 products: passes over XL, G and
# XR for their bounds, and the first product's epilogue stores the per-wave maxima of T = XL G
# ------------------------------------------------------------------------------------------------

def apply_p(XL, XR, G, prec):
    NG, B = G.shape[0], G.shape[1]
    U = torch.empty_like(G)
    ws = dash.workspace(dash.DASH_OP_APPLY, NG, B, prec, device=DEV)
    dash.dash_apply_prec(XL, XR, G, NG, B, prec, U, ws)
    return U


def apply_operands(seed, NG, B):
    """Gaussian XL and XR, and a gradient stack whose blocks differ by up to seven decades."""
    XL, XR, G = (di.gaussian((NG, B, B), seed + k) for k in range(3))
    G = (G * np.array([1.0, 3e-4, 2e3, 1e-4])[:NG, None, None]).astype(np.float32)
    return XL, XR, G


@pytest.mark.parametrize("B,NG", [(256, 4), (512, 3), (768, 2), (1024, 2)])
def test_apply_split16_matches_oracle(B, NG):
    """Several 256-wide tiles per block (T's bound is read back from every tile's waves): within
    1e-5 of the oracle's fp64 products and as accurate as the fp32 matrix cores."""
    XL, XR, G = apply_operands(490 + B, NG, B)
    U = to_host(apply_p(to_dev(XL), to_dev(XR), to_dev(G), S16))
    ref = oracle.apply(XL, G, XR)
    err = rel_err(U, ref)
    Uf = to_host(apply_p(to_dev(XL), to_dev(XR), to_dev(G), dash.DASH_FP32))
    err_f = rel_err(Uf, ref)
    print("B", B, "split16 err", err.max(), "fp32 err", err_f.max())
    assert err.max() < 1e-5
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)


def test_apply_split16_wide_magnitudes_and_identity():
    """Rows of G over six decades (D G): the small rows' pieces stay in binary16's normal range after
    the block's power of two.  Identity preconditioners: XL = I splits exactly, so U differs from G
    only by the two roundings of G and T to 22 bits (per block, at most 2^-20 of the block's
    largest element)."""
    B, NG = 256, 2
    XL, XR, G = apply_operands(495, NG, B)
    D = np.exp(di.rng(496).uniform(np.log(1e-6), 0.0, (NG, B)))
    G = (D[:, :, None] * G).astype(np.float32)
    U = to_host(apply_p(to_dev(XL), to_dev(XR), to_dev(G), S16))
    ref = oracle.apply(XL, G, XR)
    Uf = to_host(apply_p(to_dev(XL), to_dev(XR), to_dev(G), dash.DASH_FP32))
    err, err_f = rel_err(U, ref), rel_err(Uf, ref)
    print("wide split16 err", err.max(), "fp32 err", err_f.max())
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)
    I = torch.eye(B, device=DEV).expand(NG, B, B).contiguous()
    U = to_host(apply_p(I, I, to_dev(G), S16)).astype(np.float64)
    dev = np.abs(U - G).max(axis=(1, 2)) / np.abs(G).max(axis=(1, 2))
    print("identity deviation", dev)
    assert np.all(dev <= 2.0 ** -20)


@pytest.mark.parametrize("e", [-40, 40])
def test_apply_split16_equivariance_independence_and_fallback(e):
    """U(2^e XL, XR, G) = 2^e U bit for bit (XL's bound and T's maxima move by the same power of
    two); a permuted stack gives the permuted result and one block alone its result in the stack; a
    zero gradient block gives a zero block and leaves the others as they were; B = 320 has no
    256-wide tiling: the fp32 path bit for bit."""
    XL, XR, G = apply_operands(497, 4, 256)
    XLd, XRd, Gd = to_dev(XL), to_dev(XR), to_dev(G)
    U = apply_p(XLd, XRd, Gd, S16)
    assert torch.equal(apply_p(XLd * 2.0 ** e, XRd, Gd, S16), U * 2.0 ** e)
    assert torch.equal(apply_p(XLd, XRd, Gd * 2.0 ** e, S16), U * 2.0 ** e)
    perm = torch.tensor([2, 0, 3, 1], device=DEV)
    Up = apply_p(XLd[perm].contiguous(), XRd[perm].contiguous(), Gd[perm].contiguous(), S16)
    assert torch.equal(Up, U[perm])
    Ui = apply_p(XLd[1:2].contiguous(), XRd[1:2].contiguous(), Gd[1:2].contiguous(), S16)
    assert torch.equal(Ui[0], U[1])
    Gz = Gd.clone()
    Gz[2] = 0
    Uz = apply_p(XLd, XRd, Gz, S16)
    assert torch.count_nonzero(Uz[2]) == 0
    assert torch.equal(Uz[[0, 1, 3]], U[[0, 1, 3]])
    XL, XR, G = apply_operands(498, 2, 320)
    args = (to_dev(XL), to_dev(XR), to_dev(G))
    assert torch.equal(apply_p(*args, S16), apply_p(*args, dash.DASH_FP32))


# ------------------------------------------------------------------------------------------------
# Statistics L <- beta L + (1 - beta) G G^T, R <- beta R + (1 - beta) G^T G with two-piece binary16
# products (dash_update_stats_ws: G's bound per tile in the workspace)
# ------------------------------------------------------------------------------------------------

def stats_p(G, A, beta, prec):
    NG, B = G.shape[0], G.shape[1]
    ws = dash.workspace(dash.DASH_OP_STATS, NG, B, prec, device=DEV)
    dash.dash_update_stats_ws(G, NG, B, beta, prec, A, ws)


def stats_operands(seed, NG, B):
    """Gradient tiles N(0, 1e-3^2) scaled per tile over four decades, on prior statistics of the
    bench's size (G G^T / 128 + 1e-4 I, times 1e-6)."""
    G = (di.gaussian((NG, B, B), seed, 1e-3) * np.array([1.0, 1e-2, 30.0, 1e-1])[:NG, None, None]).astype(np.float32)
    L0 = (di.tiny_stack(seed=seed + 1, N=NG, B=B) * 1e-6).astype(np.float32)
    R0 = (di.tiny_stack(seed=seed + 2, N=NG, B=B) * 1e-6).astype(np.float32)
    return G, L0, R0


@pytest.mark.parametrize("B,NG", [(256, 3), (512, 2), (768, 2), (1024, 2)])
def test_stats_split16_matches_oracle(B, NG):
    """G G^T (Y's rows read as columns) and G^T G (both operands' columns gathered), triangle-only
    with the mirror: within 1e-5 of the oracle's fp64 update, as accurate as the fp32 matrix cores,
    every block exactly symmetric."""
    G, L0, R0 = stats_operands(520 + B, NG, B)
    A = to_dev(np.concatenate([L0, R0]))
    stats_p(to_dev(G), A, 0.95, S16)
    out = to_host(A)
    L_ref, R_ref = oracle.update_stats(G, 0.95, L0, R0)
    ref = np.concatenate([L_ref, R_ref])
    Af = to_dev(np.concatenate([L0, R0]))
    dash.dash_update_stats_prec(to_dev(G), NG, B, 0.95, dash.DASH_FP32, Af)
    err, err_f = rel_err(out, ref), rel_err(to_host(Af), ref)
    print("B", B, "split16 err", err.max(), "fp32 err", err_f.max())
    assert err.max() < 1e-5
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)
    assert np.array_equal(out, np.swapaxes(out, 1, 2))


@pytest.mark.parametrize("e", [-8, 8])
def test_stats_split16_equivariance_zero_tile_and_fallback(e):
    """beta = 0: L(2^e G) = 2^(2e) L(G) bit for bit (each tile's power of two moves by e and every
    piece stays as it was); a zero gradient tile leaves beta L exactly and the other tiles as they
    were; B = 320 has no 256-wide tiling: the fp32 path bit for bit."""
    NG, B = 3, 512
    G, L0, R0 = stats_operands(530, NG, B)
    Gd = to_dev(G)
    A0 = to_dev(np.concatenate([L0, R0]))
    A1, A2 = A0.clone(), A0.clone()
    stats_p(Gd, A1, 0.0, S16)
    stats_p(Gd * 2.0 ** e, A2, 0.0, S16)
    assert torch.equal(A2, A1 * 2.0 ** (2 * e))
    A3, A4 = A0.clone(), A0.clone()
    stats_p(Gd, A3, 0.95, S16)
    Gz = Gd.clone()
    Gz[1] = 0
    stats_p(Gz, A4, 0.95, S16)
    keep = [0, 2, NG, NG + 2]
    assert torch.equal(A4[keep], A3[keep])
    assert torch.equal(A4[[1, NG + 1]], A0[[1, NG + 1]] * 0.95)
    G, L0, R0 = stats_operands(531, 2, 320)
    A5, A6 = to_dev(np.concatenate([L0, R0])), to_dev(np.concatenate([L0, R0]))
    stats_p(to_dev(G), A5, 0.95, S16)
    dash.dash_update_stats(to_dev(G), 2, 320, 0.95, A6)
    assert torch.equal(A5, A6)
