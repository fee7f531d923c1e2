"""GPU parity of the solvers with split products (DASH_FP32_SPLIT): the Chebyshev solve and NDB form their fp32 products on the bfloat16 matrix cores from
exact three-piece splits of both operands.  The gates are the fp32 ones (iterate parity 1e-4
against the oracle's fp64 Clenshaw recurrence or NDB iterates, residual 1e-3), since the split
product is an fp32 product: the split is exact and the piece products it leaves out are below
fp32's own rounding.  Where the split does not apply
(Chebyshev degree 2, whose one product maps A into the recurrence's first term as it stages it; B
not a multiple of 256) the result is the fp32 path's, bit for bit."""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import (DEV, ITERATE_TOL, R_FP32, frob_scale, host_frob_scale, host_power_scale, power_scale, rel_err,
                         residual, to_dev, to_host)

pytestmark = pytest.mark.gpu

SPLIT = dash.DASH_FP32_SPLIT


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


@pytest.mark.parametrize("B,N,degrees", [(256, 4, (3, 8, 24)), (512, 2, (24,))])
def test_cheb_split_matches_oracle(B, N, degrees):
    """Several 256-wide tiles per block (B = 512: 3 of the 4 x 4 tile grid's upper triangle rows),
    power-iteration scale, the pages' interval reading hi = 1.25."""
    A, Ad = spectrum_stack(400 + B, N, B)
    s = host_power_scale(A, di.start_vectors(B, 32))
    lo, hi = 0.04, 1.25
    for d in degrees:
        X, status = cheb_p(Ad, s, d, lo, hi, SPLIT)
        Xh = to_host(X)
        ref = oracle.cheb_inverse_root(A, to_host(s), d, lo, hi)
        err = rel_err(Xh, ref)
        print("B", B, "degree", d, "split err", err.max())
        assert np.all(to_host(status) == 0)
        assert err.max() < ITERATE_TOL
        assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))  # triangle-only products, mirrored
        if d == 24:
            assert residual(Xh, A).max() < R_FP32
            # as accurate as the fp32 matrix cores on the same recurrence
            Xf, _ = cheb_p(Ad, s, d, lo, hi, dash.DASH_FP32)
            err_f = rel_err(to_host(Xf), ref)
            print("fp32 err", err_f.max())
            assert err.max() <= max(1.5 * err_f.max(), 2e-6)


def test_cheb_split_falls_back_to_fp32_bitwise():
    """Degree 2 runs one product (A mapped as it is staged, on the fp32 cores); B = 320 has no
    256-wide tiling: both equal the fp32 path bit for bit."""
    A, Ad = spectrum_stack(410, 2, 256)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 2, 0.02, 1.0, SPLIT)
    X2, _ = cheb_p(Ad, s, 2, 0.02, 1.0, dash.DASH_FP32)
    assert torch.equal(X1, X2)
    A, Ad = spectrum_stack(411, 2, 320)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 12, 0.02, 1.0, SPLIT)
    X2, _ = cheb_p(Ad, s, 12, 0.02, 1.0, dash.DASH_FP32)
    assert torch.equal(X1, X2)


def test_cheb_split_scale_equivariance_and_batch_independence():
    """A power-of-two scale of A and s moves every piece and every rounding exactly, so
    X(16 A, 16 s) = X(A, s) / 2 bit for bit; a permuted stack gives the permuted result, and one
    block alone its result in the stack."""
    A, Ad = spectrum_stack(412, 4, 256)
    s = frob_scale(Ad)
    X1, _ = cheb_p(Ad, s, 12, 0.02, 1.0, SPLIT)
    X16, _ = cheb_p(16 * Ad, 16 * s, 12, 0.02, 1.0, SPLIT)
    assert torch.equal(X16 * 2, X1)
    perm = torch.tensor([2, 0, 3, 1], device=DEV)
    Xp, _ = cheb_p(Ad[perm].contiguous(), s[perm].contiguous(), 12, 0.02, 1.0, SPLIT)
    assert torch.equal(Xp, X1[perm])
    Xi, _ = cheb_p(Ad[2:3].contiguous(), s[2:3].contiguous(), 12, 0.02, 1.0, SPLIT)
    assert torch.equal(Xi[0], X1[2])


def test_cheb_split_flags_bad_blocks():
    """A zero or NaN scale flags bit 0 and gives a NaN block; a non-finite input element (mirrored:
    the products read the upper triangle) flags bit 1; the other blocks are untouched."""
    A, Ad = spectrum_stack(413, 4, 256)
    s = frob_scale(Ad).clone()
    X_good, st_good = cheb_p(Ad, s, 8, 0.02, 1.0, SPLIT)
    assert np.all(to_host(st_good) == 0)
    s_bad = s.clone()
    s_bad[1] = 0.0
    s_bad[2] = float("nan")
    X, st = cheb_p(Ad, s_bad, 8, 0.02, 1.0, SPLIT)
    assert np.array_equal(to_host(st).astype(int) & 1, [0, 1, 1, 0])
    assert np.all(np.isnan(to_host(X)[[1, 2]]))
    assert torch.equal(X[[0, 3]], X_good[[0, 3]])
    bad = Ad.clone()
    bad[0, 3, 5] = float("inf")
    bad[0, 5, 3] = float("inf")
    Xb, stb = cheb_p(bad, s, 8, 0.02, 1.0, SPLIT)
    assert np.array_equal(to_host(stb).astype(int) & 2, [2, 0, 0, 0])
    assert torch.equal(Xb[1:], X_good[1:])


# ------------------------------------------------------------------------------------------------
# NDB with split products (dash_inverse_root_ndb_prec): every product is a general one
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
def test_ndb_split_conditioned(conditioned, scaling):
    """kappa 1e4: the stability case of the non-symmetrised NDB iteration, at the fp32 gates, and as
    accurate as the fp32 matrix cores."""
    A, Ad = conditioned
    s = host_power_scale(A, di.start_vectors(256, 32)) if scaling == "power" else host_frob_scale(A)
    T = 16 if scaling == "power" else 18
    X, _, _, status = ndb_p(Ad, s, T, T, SPLIT)
    X_ref, _, _ = oracle.ndb_inverse_root(A, to_host(s), T, T)
    err = rel_err(to_host(X), X_ref)
    Xf, _, _, _ = ndb_p(Ad, s, T, T, dash.DASH_FP32)
    err_f = rel_err(to_host(Xf), X_ref)
    print(scaling, "split err", err.max(), "fp32 err", err_f.max())
    assert err.max() < ITERATE_TOL
    assert residual(to_host(X), A).max() < R_FP32
    assert np.all(to_host(status) == 0)
    assert err.max() <= max(1.5 * err_f.max(), 2e-6)


@pytest.mark.parametrize("it1,it2", [(1, 1), (2, 3), (4, 4)])
def test_ndb_split_iterates_sqrt_and_monitor(it1, it2):
    """Several 256-wide tiles per block (B = 512, all 16 tiles): X, the square root and the monitor
    of every step against the oracle's NDB iterates."""
    A, Ad = spectrum_stack(420, 2, 512)
    s = host_frob_scale(A)
    X, R, mon, status = ndb_p(Ad, s, it1, it2, SPLIT, want_sqrt=True, want_monitor=True)
    X_ref, R_ref, mon_ref = oracle.ndb_inverse_root(A, to_host(s), it1, it2, want_sqrt=True)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(rel_err(to_host(R), R_ref)) < ITERATE_TOL
    assert np.max(np.abs(to_host(mon) - mon_ref) / mon_ref) < 1e-3
    assert np.all(to_host(status) == 0)


def test_ndb_split_fallback_equivariance_independence_and_flags(conditioned):
    """B = 320 has no 256-wide tiling: the fp32 path bit for bit.  At B = 256: X(16 A, 16 s) = X / 2
    bit for bit, one block alone equals its result in the stack, a bad scale flags bit 0 and leaves
    the other blocks untouched."""
    A, Ad = spectrum_stack(421, 2, 320)
    s = frob_scale(Ad)
    X1, _, _, _ = ndb_p(Ad, s, 5, 5, SPLIT)
    X2, _, _, _ = ndb_p(Ad, s, 5, 5, dash.DASH_FP32)
    assert torch.equal(X1, X2)
    _, Ad = conditioned
    Ad = Ad[:4].contiguous()
    s = frob_scale(Ad)
    X, _, _, _ = ndb_p(Ad, s, 8, 8, SPLIT)
    X16, _, _, _ = ndb_p(16 * Ad, 16 * s, 8, 8, SPLIT)
    assert torch.equal(X16 * 2, X)
    Xi, _, _, _ = ndb_p(Ad[3:4].contiguous(), s[3:4].contiguous(), 8, 8, SPLIT)
    assert torch.equal(Xi[0], X[3])
    s_bad = s.clone()
    s_bad[1] = float("nan")
    Xb, _, _, st = ndb_p(Ad, s_bad, 8, 8, SPLIT)
    assert np.array_equal(to_host(st).astype(int) & 1, [0, 1, 0, 0])
    assert np.all(np.isnan(to_host(Xb)[1]))
    assert torch.equal(Xb[[0, 2, 3]], X[[0, 2, 3]])


# ------------------------------------------------------------------------------------------------
# statistics (G G^T: Y's rows as columns; G^T G: both operands' columns gathered) and apply
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B", [256, 512])
def test_update_stats_split_integers_exact(B):
    """Small integers: every piece product and every sum is exact in fp32, so the split statistics
    equal the oracle's exactly, with exactly symmetric blocks."""
    NG = 2
    g = di.rng(430 + B)
    G = g.integers(-3, 4, (NG, B, B)).astype(np.float32)
    L0 = g.integers(-4, 5, (NG, B, B)).astype(np.float32)
    L0 = L0 + L0.transpose(0, 2, 1)
    R0 = g.integers(-4, 5, (NG, B, B)).astype(np.float32)
    R0 = R0 + R0.transpose(0, 2, 1)
    A = to_dev(np.concatenate([L0, R0]))
    dash.dash_update_stats_prec(to_dev(G), NG, B, 0.5, SPLIT, A)
    out = to_host(A)
    L_ref, R_ref = oracle.update_stats(G, 0.5, L0, R0)
    assert np.array_equal(out[:NG], L_ref) and np.array_equal(out[NG:], R_ref)


def test_update_stats_split_gaussian():
    NG, B = 3, 512
    G = di.gaussian((NG, B, B), 440, 1e-3)
    L0 = di.tiny_stack(seed=441, N=NG, B=B) * 1e-6
    R0 = di.tiny_stack(seed=442, N=NG, B=B) * 1e-6
    A = to_dev(np.concatenate([L0, R0]))
    dash.dash_update_stats_prec(to_dev(G), NG, B, 0.95, SPLIT, A)
    out = to_host(A)
    L_ref, R_ref = oracle.update_stats(G, 0.95, L0, R0)
    assert np.max(rel_err(out[:NG], L_ref)) < 1e-5 and np.max(rel_err(out[NG:], R_ref)) < 1e-5
    assert np.array_equal(out, out.transpose(0, 2, 1))


@pytest.mark.parametrize("B", [256, 512, 320])
def test_apply_split_matches_oracle(B):
    """General operands on both products; B = 320 runs the fp32 matrix cores (bit for bit the fp32
    path)."""
    NG = 3
    XL, XR, G = (di.gaussian((NG, B, B), seed) for seed in (450, 451, 452))
    U = torch.empty((NG, B, B), device=DEV)
    ws = dash.workspace(dash.DASH_OP_APPLY, NG, B, SPLIT, device=DEV)
    dash.dash_apply_prec(to_dev(XL), to_dev(XR), to_dev(G), NG, B, SPLIT, U, ws)
    U_ref = oracle.apply(XL, G, XR)
    assert np.max(rel_err(to_host(U), U_ref)) < 1e-5
    if B % 256:
        U2 = torch.empty_like(U)
        dash.dash_apply(to_dev(XL), to_dev(XR), to_dev(G), NG, B, U2, ws)
        assert torch.equal(U, U2)
    # identity preconditioners pass the gradient through exactly (pieces of 1 and 0 are exact)
    I = torch.eye(B, device=DEV).expand(NG, B, B).contiguous()
    dash.dash_apply_prec(I, I, to_dev(G), NG, B, SPLIT, U, ws)
    assert np.array_equal(to_host(U), G.astype(np.float64))


# ------------------------------------------------------------------------------------------------
# Coupled Newton in fp32 with split products (every product but the M S^4 launches that also write
# S_{k+1})
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("scaling", ["power", "frobenius"])
def test_cn_split_conditioned(conditioned, scaling):
    A, Ad = conditioned
    s = host_power_scale(A, di.start_vectors(256, 32)) if scaling == "power" else host_frob_scale(A)
    T = 16
    N = Ad.shape[0]
    X = torch.empty_like(Ad)
    mon = torch.empty((N, T), device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CN, N, 256, SPLIT, device=DEV)
    dash.dash_inverse_root_cn(Ad, s, N, 256, 4, T, SPLIT, X, monitor=mon, status=status, ws=ws)
    X_ref, mon_ref = oracle.cn_inverse_root(A, to_host(s), T)
    err = rel_err(to_host(X), X_ref)
    print(scaling, "CN split err", err.max())
    assert err.max() < ITERATE_TOL
    assert residual(to_host(X), A).max() < R_FP32
    assert np.all(to_host(status) == 0)
    m = to_host(mon)
    assert np.max(np.abs(m[:, :4] - mon_ref[:, :4]) / mon_ref[:, :4]) < 1e-3


def test_cn_split_fallback_bitwise():
    """B = 320 has no 256-wide tiling: the fp32 path bit for bit."""
    A, Ad = spectrum_stack(460, 2, 320)
    s = frob_scale(Ad)
    out = []
    for prec in (SPLIT, dash.DASH_FP32):
        X = torch.empty_like(Ad)
        ws = dash.workspace(dash.DASH_OP_CN, 2, 320, prec, device=DEV)
        dash.dash_inverse_root_cn(Ad, s, 2, 320, 4, 6, prec, X, ws=ws)
        out.append(X)
    assert torch.equal(out[0], out[1])


# ------------------------------------------------------------------------------------------------
# power-iteration scale with split products (the streaming step, B % 128 == 0)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,N", [(128, 3), (256, 3), (1024, 2)])
def test_power_scale_split_matches_oracle(B, N):
    """The streaming step's products from three-piece bfloat16 splits: s against the oracle's fp64
    power iteration at the fp32 gate, and within 2e-6 of the fp32 matrix cores' s; k = 5 leaves 27
    zero columns of the iterate."""
    A, Ad = spectrum_stack(700 + B, N, B)
    for k in (32, 5):
        V0 = di.start_vectors(B, k)
        s = to_host(power_scale(Ad, to_dev(V0), 10, SPLIT))
        s_ref, _ = oracle.mpi(A, V0, 10)
        s32 = to_host(power_scale(Ad, to_dev(V0), 10, dash.DASH_FP32))
        print("B", B, "k", k, "split rel err", np.max(np.abs(s - s_ref) / s_ref))
        assert np.max(np.abs(s - s_ref) / s_ref) < 1e-5
        assert np.max(np.abs(s - s32) / s32) < 2e-6


def test_power_scale_split_conditioned_and_fallback(conditioned):
    """kappa 1e4 at B = 256 against the oracle; B = 192 (no 128-row blocks) runs the fp32 step, bit
    for bit."""
    A, Ad = conditioned
    V0 = di.start_vectors(256, 32)
    s = to_host(power_scale(Ad, to_dev(V0), 10, SPLIT))
    s_ref, _ = oracle.mpi(A, V0, 10)
    assert np.max(np.abs(s - s_ref) / s_ref) < 1e-5
    A2, Ad2 = spectrum_stack(790, 2, 192)
    V2 = to_dev(di.start_vectors(192, 32))
    assert torch.equal(power_scale(Ad2, V2, 10, SPLIT), power_scale(Ad2, V2, 10, dash.DASH_FP32))


def test_power_scale_split_equivariance_and_independence():
    """s(4 A) = 4 s(A) bitwise (the split of 4 x is 4 times the split of x), and a block alone gives
    the s it gets inside a stack."""
    A, Ad = spectrum_stack(795, 3, 256)
    V0 = to_dev(di.start_vectors(256, 32))
    s1 = power_scale(Ad, V0, 10, SPLIT)
    s4 = power_scale(4.0 * Ad, V0, 10, SPLIT)
    assert torch.equal(s4, 4.0 * s1)
    assert torch.equal(power_scale(Ad[1:2].contiguous(), V0, 10, SPLIT), s1[1:2])
