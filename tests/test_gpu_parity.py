"""GPU parity of every hot-path call against the CPU oracle, on the tiny (4 x 64 x 64) and the
conditioned (16 x 256 x 256, kappa 1e4) stacks, plus ragged tile shapes and edge cases.

Gates: fp32 iterate parity max_i ||X_gpu - X_oracle||_F / ||X_oracle||_F <= 1e-4 with the SAME scale
s fed to both sides; residual ||X^4 A - I||_F / sqrt(B) <= 1e-3 (fp32) and <= 5e-3 (fp16 operands)
evaluated in fp64 on the host.
"""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import (DEV, ITERATE_TOL, R_FP16, R_FP32, cheb, cn, frob_scale, host_frob_scale, host_power_scale,
                         ndb, power_scale, rel_err,
                         residual, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    A = di.tiny_stack()
    return A, to_dev(A)


@pytest.fixture(scope="module")
def conditioned():
    A, Q, lam = di.conditioned_stack()
    return A, to_dev(A)


# ------------------------------------------------------------------------------------------------
# scaling
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("k,steps", [(32, 10), (7, 3), (1, 1), (32, 1)])
def test_power_scale_tiny(tiny, k, steps):
    A, Ad = tiny
    V0 = di.start_vectors(A.shape[1], k)
    s = to_host(power_scale(Ad, to_dev(V0), steps))
    s_ref, _ = oracle.mpi(A, V0, steps)
    assert np.max(np.abs(s - s_ref) / s_ref) < 1e-5


def test_power_scale_conditioned_fp32_and_fp16(conditioned):
    A, Ad = conditioned
    V0 = di.start_vectors(256, 32)
    s = to_host(power_scale(Ad, to_dev(V0), 10))
    s_ref, _ = oracle.mpi(A, V0, 10)
    assert np.max(np.abs(s - s_ref) / s_ref) < 1e-5
    s16 = to_host(power_scale(Ad, to_dev(V0), 10, dash.DASH_FP16))
    s16_ref, _ = oracle.mpi(A, V0, 10, half=True)
    assert np.max(np.abs(s16 - s16_ref) / s16_ref) < 2e-3
    assert np.max(np.abs(s16 - s_ref) / s_ref) < 2e-3


@pytest.mark.parametrize("B", [64, 128, 192, 320])
def test_power_scale_ring_depths(B):
    """k-loops of 1, 2 and 4 register-ring slices (fp32 slices are 32 wide, binary16 slices 64) on
    64- and 128-row workgroups; k = 5 start vectors leave 27 zero columns."""
    A64, _, _ = di.known_spectrum_stack(150 + B, 2, B, 0.05, 1.0)
    A = A64.astype(np.float32)
    for k in (32, 5):
        V0 = di.start_vectors(B, k)
        s = to_host(power_scale(to_dev(A), to_dev(V0), 10))
        s_ref, _ = oracle.mpi(A, V0, 10)
        assert np.max(np.abs(s - s_ref) / s_ref) < 1e-5
        s16 = to_host(power_scale(to_dev(A), to_dev(V0), 10, dash.DASH_FP16))
        s16_ref, _ = oracle.mpi(A, V0, 10, half=True)
        assert np.max(np.abs(s16 - s16_ref) / s16_ref) < 2e-3


def test_frobenius(tiny, conditioned):
    for A, Ad in (tiny, conditioned):
        s = to_host(frob_scale(Ad))
        assert np.max(np.abs(s - oracle.frobenius(A)) / oracle.frobenius(A)) < 1e-6


# ------------------------------------------------------------------------------------------------
# Newton-Denman-Beavers
# ------------------------------------------------------------------------------------------------

def test_ndb_tiny_full_stack(tiny):
    A, Ad = tiny
    V0 = di.start_vectors(64, 32)
    s = host_power_scale(A, V0)
    X, R, mon, status = ndb(Ad, s, 20, 20, want_sqrt=True, want_monitor=True)
    s_h = to_host(s)
    X_ref, R_ref, mon_ref = oracle.ndb_inverse_root(A, s_h, 20, 20, want_sqrt=True)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(rel_err(to_host(R), R_ref)) < ITERATE_TOL
    assert np.max(residual(to_host(X), A)) < R_FP32
    assert np.all(to_host(status) == 0)
    m = to_host(mon)
    big = mon_ref > 1e-3  # below that the monitor is at fp32 rounding level
    assert np.max(np.abs(m[big] - mon_ref[big]) / mon_ref[big]) < 1e-3
    assert np.all(m[~big] < 2e-3)


@pytest.mark.parametrize("scaling", ["power", "frobenius"])
def test_ndb_conditioned(conditioned, scaling):
    A, Ad = conditioned
    s = host_power_scale(A, di.start_vectors(256, 32)) if scaling == "power" else host_frob_scale(A)
    T = 16 if scaling == "power" else 18
    X, _, _, status = ndb(Ad, s, T, T)
    X_ref, _, _ = oracle.ndb_inverse_root(A, to_host(s), T, T)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(residual(to_host(X), A)) < R_FP32
    assert np.all(to_host(status) == 0)


@pytest.mark.parametrize("it1,it2", [(1, 1), (1, 3), (2, 1), (3, 2)])
def test_ndb_few_steps_match_oracle_iterates(tiny, it1, it2):
    A, Ad = tiny
    s = host_frob_scale(A)
    X, R, mon, _ = ndb(Ad, s, it1, it2, want_sqrt=True, want_monitor=True)
    X_ref, R_ref, mon_ref = oracle.ndb_inverse_root(A, to_host(s), it1, it2, want_sqrt=True)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(rel_err(to_host(R), R_ref)) < ITERATE_TOL
    assert np.max(np.abs(to_host(mon) - mon_ref) / mon_ref) < 1e-3


# ------------------------------------------------------------------------------------------------
# Coupled Newton
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("scaling", ["power", "frobenius"])
def test_cn_conditioned(conditioned, scaling):
    A, Ad = conditioned
    s = host_power_scale(A, di.start_vectors(256, 32)) if scaling == "power" else host_frob_scale(A)
    T = 16
    X, mon, status = cn(Ad, s, T, want_monitor=True)
    X_ref, mon_ref = oracle.cn_inverse_root(A, to_host(s), T)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(residual(to_host(X), A)) < R_FP32
    assert np.all(to_host(status) == 0)
    # the monitor ||M_k - I||/sqrt(B) differences O(1) fp32 entries: near convergence its error has
    # an absolute floor of fp32 rounding accumulated in M over the steps
    m = to_host(mon)
    assert np.all(np.abs(m - mon_ref) <= 1e-3 * mon_ref + 2e-5)


@pytest.mark.parametrize("iters", [1, 2, 3, 6])
def test_cn_few_steps_match_oracle_iterates(tiny, iters):
    A, Ad = tiny
    s = host_power_scale(A, di.start_vectors(64, 32))
    X, mon, _ = cn(Ad, s, iters, want_monitor=True)
    X_ref, mon_ref = oracle.cn_inverse_root(A, to_host(s), iters)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(np.abs(to_host(mon) - mon_ref) / mon_ref) < 1e-3


def test_cn_fp16_tiny(tiny):
    A, Ad = tiny
    s = host_power_scale(A, di.start_vectors(64, 32))
    X, _, status = cn(Ad, s, 8, dash.DASH_FP16)
    Xh = to_host(X)
    assert np.max(residual(Xh, A)) < R_FP16
    X_emul, _ = oracle.cn_inverse_root(A, to_host(s), 8, half_storage=True)
    assert np.max(rel_err(Xh, X_emul)) < 5e-3
    assert np.all(to_host(status) == 0)


@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP16])
def test_cn_reads_only_the_upper_triangle(prec):
    """CN builds its start terms from the upper triangle of A: garbage below the diagonal is ignored."""
    A64, _, _ = di.known_spectrum_stack(130, 2, 256, 0.2, 1.0)
    A = A64.astype(np.float32)
    noisy = A.copy()
    low = np.tril_indices(256, -1)
    noisy[:, low[0], low[1]] += di.gaussian((2, len(low[0])), 131, 0.05)
    s = torch.ones(2, device=DEV)
    X_clean, _, _ = cn(to_dev(A), s, 6, prec)
    X_noisy, _, _ = cn(to_dev(noisy), s, 6, prec)
    assert torch.equal(X_clean, X_noisy)
    Xh = to_host(X_noisy)
    if prec == dash.DASH_FP16:  # triangle-only products: exactly symmetric
        assert np.array_equal(Xh, Xh.transpose(0, 2, 1))
    else:
        assert np.max(np.abs(Xh - Xh.transpose(0, 2, 1))) < 1e-5 * np.abs(Xh).max()


@pytest.mark.parametrize("iters", [2, 3])
def test_cn_fp16_short_runs(tiny, iters):
    """T = 2 and 3: the first iterate X_1 = S_0 enters the last and the dual products directly."""
    A, Ad = tiny
    s = host_power_scale(A, di.start_vectors(64, 32))
    X, _, status = cn(Ad, s, iters, dash.DASH_FP16)
    X_emul, _ = oracle.cn_inverse_root(A, to_host(s), iters, half_storage=True)
    assert np.max(rel_err(to_host(X), X_emul)) < 5e-3
    assert np.all(to_host(status) == 0)


@pytest.mark.parametrize("B", [128, 192, 256, 512])
def test_cn_fp16_wide_tiles(B):
    """B % 256 == 0 runs the 256 x 256 fp16 product tile, 128 and 192 the 128/64 tiles; compare with
    the binary16-storage oracle."""
    A64, _, _ = di.known_spectrum_stack(120 + B, 3, B, 0.2, 1.0)  # kappa 5, like the Gram stacks
    A = A64.astype(np.float32)
    Ad = to_dev(A)
    s = host_power_scale(A, di.start_vectors(B, 32))
    X, mon, status = cn(Ad, s, 9, dash.DASH_FP16, want_monitor=True)
    Xh = to_host(X)
    assert np.max(residual(Xh, A)) < R_FP16
    X_emul, mon_ref = oracle.cn_inverse_root(A, to_host(s), 9, half_storage=True)
    assert np.max(rel_err(Xh, X_emul)) < 5e-3
    assert np.all(to_host(status) == 0)
    m = to_host(mon)
    assert np.max(np.abs(m[:, :4] - mon_ref[:, :4]) / mon_ref[:, :4]) < 1e-2


# ------------------------------------------------------------------------------------------------
# Chebyshev / Clenshaw
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("degree", [1, 2, 3, 8, 24])
def test_cheb_tiny(tiny, degree):
    A, Ad = tiny
    s = host_power_scale(A, di.start_vectors(64, 32))
    lo, hi = 0.02, 1.25
    X, status = cheb(Ad, s, degree, lo, hi)
    X_ref = oracle.cheb_inverse_root(A, to_host(s), degree, lo, hi)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.all(to_host(status) == 0)


def test_cheb_known_spectrum_accuracy():
    A64, Q, lam = di.known_spectrum_stack(81, 4, 128, 0.05, 1.0)
    A = A64.astype(np.float32)
    Ad = to_dev(A)
    s = torch.ones(4, device=DEV)
    X, _ = cheb(Ad, s, 24, 0.04, 1.1)
    X_ref = oracle.cheb_inverse_root(A, 1.0, 24, 0.04, 1.1)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.max(residual(to_host(X), A)) < R_FP32


# ------------------------------------------------------------------------------------------------
# statistics, apply, stacking (ragged tile shapes: B = 64, 192, 320 use the 64-wide tiles)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B", [64, 128, 192, 320])
def test_apply_matches_oracle(B):
    NG = 3
    XL, XR, G = (di.gaussian((NG, B, B), seed) for seed in (91, 92, 93))
    U = torch.empty((NG, B, B), device=DEV)
    ws = dash.workspace(dash.DASH_OP_APPLY, NG, B, device=DEV)
    dash.dash_apply(to_dev(XL), to_dev(XR), to_dev(G), NG, B, U, ws)
    U_ref = oracle.apply(XL, G, XR)
    assert np.max(rel_err(to_host(U), U_ref)) < 1e-5


def test_apply_identity_is_exact():
    NG, B = 2, 128
    G = di.gaussian((NG, B, B), 94)
    I = torch.eye(B, device=DEV).expand(NG, B, B).contiguous()
    U = torch.empty((NG, B, B), device=DEV)
    ws = dash.workspace(dash.DASH_OP_APPLY, NG, B, device=DEV)
    dash.dash_apply(I, I, to_dev(G), NG, B, U, ws)
    assert np.array_equal(to_host(U), G.astype(np.float64))


@pytest.mark.parametrize("B", [64, 192, 256])
def test_update_stats_integers_exact_and_symmetric(B):
    NG = 2
    g = di.rng(95)
    G = g.integers(-3, 4, (NG, B, B)).astype(np.float32)
    L0 = g.integers(-4, 5, (NG, B, B)).astype(np.float32)
    L0 = L0 + L0.transpose(0, 2, 1)
    R0 = g.integers(-4, 5, (NG, B, B)).astype(np.float32)
    R0 = R0 + R0.transpose(0, 2, 1)
    A = to_dev(np.concatenate([L0, R0]))
    dash.dash_update_stats(to_dev(G), NG, B, 0.5, A)
    out = to_host(A)
    L_ref, R_ref = oracle.update_stats(G, 0.5, L0, R0)
    assert np.array_equal(out[:NG], L_ref) and np.array_equal(out[NG:], R_ref)


def test_update_stats_gaussian():
    NG, B = 3, 256
    G = di.gaussian((NG, B, B), 96, 1e-3)
    L0 = di.tiny_stack(seed=97, N=NG, B=B) * 1e-6
    R0 = di.tiny_stack(seed=98, N=NG, B=B) * 1e-6
    A = to_dev(np.concatenate([L0, R0]))
    dash.dash_update_stats(to_dev(G), NG, B, 0.95, A)
    out = to_host(A)
    L_ref, R_ref = oracle.update_stats(G, 0.95, L0, R0)
    assert np.max(rel_err(out[:NG], L_ref)) < 1e-5 and np.max(rel_err(out[NG:], R_ref)) < 1e-5
    assert np.array_equal(out, out.transpose(0, 2, 1))


def test_stack_unstack_round_trip():
    B = 64
    shapes = [(128, 192), (64, 64), (192, 128)]
    W = [di.gaussian(s, 100 + i) for i, s in enumerate(shapes)]
    Wd = [to_dev(w) for w in W]
    n = di.num_tiles(shapes, B)
    S = torch.empty((n, B, B), device=DEV)
    dash.dash_stack(Wd, B, S)
    assert np.array_equal(to_host(S), oracle.stack(W, B).astype(np.float64))
    outs = [torch.zeros(s, device=DEV) for s in shapes]
    dash.dash_unstack(S, B, outs)
    for o, w in zip(outs, W):
        assert np.array_equal(to_host(o), w.astype(np.float64))


@pytest.mark.parametrize("B", [64, 192])
def test_stack_many_weights(B):
    # 37 weights: more than one launch takes (32); with B = 192 a workgroup's chunk of the stack
    # straddles tile rows and tiles.  Unstack writes into strided views; the rest stays untouched.
    shapes = [(B * (1 + i % 3), B * (1 + (i * 7) % 4)) for i in range(37)]
    W = [di.gaussian(s, 200 + i) for i, s in enumerate(shapes)]
    n = di.num_tiles(shapes, B)
    S = torch.empty((n, B, B), device=DEV)
    dash.dash_stack([to_dev(w) for w in W], B, S)
    assert np.array_equal(to_host(S), oracle.stack(W, B).astype(np.float64))
    bigs = [torch.full((r, c + 64), -7.0, device=DEV) for r, c in shapes]
    dash.dash_unstack(S, B, [b[:, 32:32 + c] for b, (r, c) in zip(bigs, shapes)])
    for b, w, (r, c) in zip(bigs, W, shapes):
        h = to_host(b)
        assert np.array_equal(h[:, 32:32 + c], w.astype(np.float64))
        assert np.all(h[:, :32] == -7.0) and np.all(h[:, 32 + c:] == -7.0)


def _views(shapes, fill, pad=8):
    """Device views of the given shapes with a 16-byte-aligned leading dimension and room around them."""
    bigs, views = [], []
    for r, c in shapes:
        ld = (c + 3) // 4 * 4 + pad
        big = torch.full((r + 2, ld + 8), fill, device=DEV)
        bigs.append(big)
        views.append(big[1:1 + r, 4:4 + c])
    return bigs, views


def test_stack_edge_tiles():
    """Sides that are not multiples of B: zero-padded edge tiles, weights smaller than a tile,
    strided views; unstack writes the weight and nothing else."""
    B = 64
    shapes = [(100, 70), (3, 5), (64, 130), (200, 4), (130, 257), (64, 64)]
    W = [di.gaussian(s, 300 + i) for i, s in enumerate(shapes)]
    _, src = _views(shapes, 0.0)
    for v, w in zip(src, W):
        v.copy_(to_dev(w))
    n = di.num_tiles(shapes, B)
    S = torch.full((n, B, B), 5.0, device=DEV)  # padding must be written as zeros
    dash.dash_stack(src, B, S)
    assert np.array_equal(to_host(S), oracle.stack(W, B).astype(np.float64))
    bigs, dst = _views(shapes, -7.0)
    dash.dash_unstack(S, B, dst)
    for big, w, (r, c) in zip(bigs, W, shapes):
        h = to_host(big)
        assert np.array_equal(h[1:1 + r, 4:4 + c], w.astype(np.float64))
        h[1:1 + r, 4:4 + c] = -7.0
        assert np.all(h == -7.0)


def test_edge_tiles_through_the_step():
    """A Shampoo step on weights with edge tiles (stack, statistics over damped L/R, Frobenius scale,
    NDB, apply, unstack) against the oracle's same steps."""
    B = 64
    shapes = [(100, 70), (64, 130)]
    W = [di.gaussian(s, 320 + i) for i, s in enumerate(shapes)]
    NG = di.num_tiles(shapes, B)
    _, src = _views(shapes, 0.0)
    for v, w in zip(src, W):
        v.copy_(to_dev(w))
    G = torch.empty((NG, B, B), device=DEV)
    dash.dash_stack(src, B, G)
    damp = np.broadcast_to(0.05 * np.eye(B), (NG, B, B)).astype(np.float32)
    A = to_dev(np.concatenate([damp, damp]))
    dash.dash_update_stats(G, NG, B, 0.5, A)
    s = frob_scale(A)
    X, _, _, _ = ndb(A, s, 8, 8)
    U = torch.empty_like(G)
    dash.dash_apply(X[:NG].contiguous(), X[NG:].contiguous(), G, NG, B, U,
                    ws=dash.workspace(dash.DASH_OP_APPLY, NG, B, device=DEV))
    _, dst = _views(shapes, 0.0)
    dash.dash_unstack(U, B, dst)
    G_ref = oracle.stack(W, B).astype(np.float64)
    L_ref, R_ref = oracle.update_stats(G_ref, 0.5, damp.astype(np.float64), damp.astype(np.float64))
    A_ref = np.concatenate([L_ref, R_ref])
    assert np.max(rel_err(to_host(A), A_ref)) < 1e-6
    s_ref = oracle.frobenius(A_ref)  # the oracle's own pipeline, on its own statistics and scale
    assert np.max(np.abs(to_host(s) - s_ref) / s_ref) < 1e-6
    X_ref, _, _ = oracle.ndb_inverse_root(A_ref, s_ref, 8, 8)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    U_ref = oracle.unstack(oracle.apply(X_ref[:NG], G_ref, X_ref[NG:]), shapes, B)
    for v, u in zip(dst, U_ref):
        assert np.max(rel_err(to_host(v), u)) < ITERATE_TOL


def test_stack_strided_rows():
    B = 64
    big = to_dev(di.gaussian((128, 256), 110))
    view = big[:, 64:192]  # ld = 256, cols = 128
    S = torch.empty((4, B, B), device=DEV)
    dash.dash_stack([view], B, S)
    assert np.array_equal(to_host(S), oracle.stack([to_host(view)], B))


# ------------------------------------------------------------------------------------------------
# invariants: scale equivariance, batch independence, determinism, per-block failure reporting
# ------------------------------------------------------------------------------------------------

def test_scale_equivariance_bitwise(tiny):
    A, Ad = tiny
    s = frob_scale(Ad)
    X1, _, _, _ = ndb(Ad, s, 6, 6)
    X16, _, _, _ = ndb(16 * Ad, 16 * s, 6, 6)
    assert torch.equal(X16 * 2, X1)
    C1, _, _ = cn(Ad, s, 6)
    C16, _, _ = cn(16 * Ad, 16 * s, 6)
    assert torch.equal(C16 * 2, C1)
    H1, _ = cheb(Ad, s, 12, 0.02, 1.25)
    H16, _ = cheb(16 * Ad, 16 * s, 12, 0.02, 1.25)
    assert torch.equal(H16 * 2, H1)
    # binary16 operands: a power-of-two scale shifts every rounding exactly, through the
    # power-of-two prescale of the half-precision power iteration too
    V0 = to_dev(di.start_vectors(64, 32))
    p1 = power_scale(Ad, V0, 10, dash.DASH_FP16)
    p16 = power_scale(16 * Ad, V0, 10, dash.DASH_FP16)
    assert torch.equal(p16, 16 * p1)
    F1, _, _ = cn(Ad, p1, 6, dash.DASH_FP16)
    F16, _, _ = cn(16 * Ad, p16, 6, dash.DASH_FP16)
    assert torch.equal(F16 * 2, F1)


def test_batch_independence_and_determinism(conditioned):
    _, Ad = conditioned
    s = frob_scale(Ad)
    X, _, _, _ = ndb(Ad, s, 8, 8)
    X2, _, _, _ = ndb(Ad, s, 8, 8)
    assert torch.equal(X, X2)
    for i in (0, 7, 15):
        Xi, _, _, _ = ndb(Ad[i:i + 1].contiguous(), s[i:i + 1].contiguous(), 8, 8)
        assert torch.equal(Xi[0], X[i])
    perm = torch.tensor([3, 1, 15, 0, 2, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14], device=DEV)
    Xp, _, _ = cn(Ad[perm].contiguous(), s[perm].contiguous(), 6)
    Xc, _, _ = cn(Ad, s, 6)
    assert torch.equal(Xp, Xc[perm])
    Hp, _, _ = cn(Ad[perm].contiguous(), s[perm].contiguous(), 6, dash.DASH_FP16)
    Hc, _, _ = cn(Ad, s, 6, dash.DASH_FP16)
    assert torch.equal(Hp, Hc[perm])
    Cp, _ = cheb(Ad[perm].contiguous(), s[perm].contiguous(), 16, 0.01, 1.25)
    Cc, _ = cheb(Ad, s, 16, 0.01, 1.25)
    assert torch.equal(Cp, Cc[perm])


def test_stack_slices_solve_like_the_whole_stack(conditioned):
    """Round-robin refresh at update frequency f > 1 passes a slice of the stack (a pointer offset)
    to the scale and the solver: the slice's roots equal the whole stack's for those blocks, bit for
    bit, and the blocks outside the slice are left untouched."""
    A, Ad = conditioned
    N, B = Ad.shape[0], Ad.shape[1]
    V0 = to_dev(di.start_vectors(B, 32))
    s_all = power_scale(Ad, V0, 10)
    X_all, _ = cheb(Ad, s_all, 12, 0.01, 1.25)
    f = 4
    n = N // f
    X = torch.full_like(Ad, 7.0)
    s = torch.zeros(N, device=DEV)
    ws_s = dash.workspace(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 32, device=DEV)
    ws_c = dash.workspace(dash.DASH_OP_CHEB, N, B, device=DEV)
    for i in (1, 3):
        o = i * n
        dash.dash_scale(Ad[o:o + n], n, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, V0, s[o:o + n], ws_s)
        dash.dash_inverse_root_cheb(Ad[o:o + n], s[o:o + n], n, B, 12, 0.01, 1.25, X[o:o + n], ws=ws_c)
        assert torch.equal(s[o:o + n], s_all[o:o + n])
        assert torch.equal(X[o:o + n], X_all[o:o + n])
    for i in (0, 2):
        assert bool((X[i * n:(i + 1) * n] == 7.0).all())


def test_bad_blocks_are_flagged_and_isolated(tiny):
    A, Ad = tiny
    s = frob_scale(Ad).clone()
    s[1] = 0.0
    s[2] = float("nan")
    X, _, _, status = ndb(Ad, s, 6, 6)
    st = to_host(status).astype(int)
    Xh = to_host(X)
    assert st[0] == 0 and st[3] == 0
    assert st[1] & 1 and st[2] & 1
    assert np.all(np.isnan(Xh[1])) and np.all(np.isnan(Xh[2]))
    X_ok, _, _, _ = ndb(Ad[[0, 3]].contiguous(), s[[0, 3]].contiguous(), 6, 6)
    assert np.array_equal(to_host(X_ok), Xh[[0, 3]])
    Xc, _, stc = cn(Ad, s, 5)
    assert np.array_equal(to_host(stc).astype(int) & 1, [0, 1, 1, 0])
    Xh, sth = cheb(Ad, s, 8, 0.02, 1.25)
    assert np.array_equal(to_host(sth).astype(int) & 1, [0, 1, 1, 0])
    Xf, _, stf = cn(Ad, s, 5, dash.DASH_FP16)
    assert np.array_equal(to_host(stf).astype(int) & 1, [0, 1, 1, 0])
    assert np.all(np.isnan(to_host(Xf)[[1, 2]]))
    # a non-finite input block: flagged as a non-finite output, neighbours untouched
    bad = Ad.clone()
    bad[0, 3, 5] = float("inf")
    bad[0, 5, 3] = float("inf")  # CN and Chebyshev read the upper triangle only
    s_ok = frob_scale(Ad)
    _, _, _, st2 = ndb(bad, s_ok, 4, 4)
    assert np.array_equal(to_host(st2).astype(int) & 2, [2, 0, 0, 0])
    X_good, _, _ = cn(Ad, s_ok, 5)
    for prec in (dash.DASH_FP32, dash.DASH_FP16):
        Xb, _, stb = cn(bad, s_ok, 5, prec)
        assert np.array_equal(to_host(stb).astype(int) & 2, [2, 0, 0, 0])
        if prec == dash.DASH_FP32:
            assert torch.equal(Xb[1:], X_good[1:])
    Hb, sth2 = cheb(bad, s_ok, 8, 0.02, 1.25)
    assert np.array_equal(to_host(sth2).astype(int) & 2, [2, 0, 0, 0])
    # a non-finite block gives a non-finite power-iteration scale; the solver then flags bit 0
    s_bad = power_scale(bad, to_dev(di.start_vectors(64, 32)), 10)
    assert not np.isfinite(to_host(s_bad)[0]) and np.all(np.isfinite(to_host(s_bad)[1:]))


def test_c2_steps_to_tolerance():
    """Steps to reach the residual 1e-3 on every block of the kappa 1e4 stack, for NDB and CN after
    power-iteration and Frobenius scaling (the counts bench.py --only c2 reports): every count is
    reached, and the oracle's fp64 iteration with its own scale agrees to one step (it has not
    converged two steps earlier and has one step later)."""
    import importlib.util
    import os

    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    res = bench.c2_steps_to_tolerance(dash, di, torch, DEV)
    A = di.conditioned_stack()[0]
    scales = {"power": oracle.mpi(A.astype(np.float64), di.start_vectors(256, 32), 10)[0],
              "frobenius": oracle.frobenius(A.astype(np.float64))}
    for key, rec in res.items():
        if not isinstance(rec, dict):
            continue
        solver, name = key.split("_")
        T = rec["steps"]
        assert T is not None and rec["residual"] <= 1e-3, key
        s = scales[name]

        def oracle_residual(t):
            if solver == "ndb":
                X, _, _ = oracle.ndb_inverse_root(A, s, t, t)
            else:
                X, _ = oracle.cn_inverse_root(A, s, t)
            return residual(X, A).max()

        if T >= 3:
            assert oracle_residual(T - 2) > 1e-3, key
        assert oracle_residual(T + 1) <= 1e-3, key
