"""GPU checks at the full benchmark size (N=3072 blocks of 1024 x 1024, the launch configuration that
bench.py times): sampled blocks against the oracle one by one, plus properties that hold for every
block (the residual ||X^4 A - I||_F / sqrt(B), checked on the GPU with torch products)."""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import DEV, ITERATE_TOL, R_FP16, R_FP32, rel_err, residual

pytestmark = pytest.mark.gpu

B = 1024
SHAPES = di.llama_weight_shapes()
NG = di.num_tiles(SHAPES, B)
N = 2 * NG
SAMPLE = [0, 1535, 1536, 3071]       # first/last L block, first/last R block
ORACLE_SAMPLE = [17, 2900]            # blocks recomputed by the fp64 oracle


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def residual_all(X, A, chunk=128):
    """max over all blocks of ||X^4 A - I||_F / sqrt(B), computed with torch fp32 products."""
    worst = 0.0
    eye = torch.eye(B, device=DEV)
    for i in range(0, X.shape[0], chunk):
        x = X[i:i + chunk]
        x2 = torch.matmul(x, x)
        r = torch.matmul(torch.matmul(x2, x2), A[i:i + chunk]) - eye
        worst = max(worst, float((torch.linalg.matrix_norm(r) / B ** 0.5).max()))
        del x2, r
    return worst


@pytest.fixture(scope="module")
def stack():
    A = di.gram_stack_torch(N, B, seed=di.SEED_GRAM, device=DEV)
    V0 = torch.from_numpy(di.start_vectors(B, 32)).to(DEV)
    yield A, V0
    del A
    torch.cuda.empty_cache()


def tile_of(grads, t):
    """Tile t of the stacking order (weight-major, then tile row, then tile column), read from the
    weights on the host."""
    for w in grads:
        r, c = w.shape
        n = (r // B) * (c // B)
        if t < n:
            tr, tc = divmod(t, c // B)
            return host(w[tr * B:(tr + 1) * B, tc * B:(tc + 1) * B])
        t -= n
    raise IndexError(t)


def scale(A, V0, prec):
    s = torch.empty(N, device=DEV)
    ws = dash.workspace(dash.DASH_OP_SCALE, N, B, prec, 32, device=DEV)
    dash.dash_scale(A, N, B, dash.DASH_SCALE_POWER, prec, 32, 10, V0, s, ws)
    return s


def pinned_scale(A, V0, prec, idx, tol, half=False):
    """The GPU scale of every block, checked on the blocks idx against the oracle's power iteration
    (relative tol), whose values, rounded to fp32, then replace the GPU's there: the solve and the
    oracle take the same scale on those blocks, and it comes from the oracle.  Returns (s on the
    device, the oracle's fp32 scale of idx in fp64)."""
    s = scale(A, V0, prec)
    s_ref, _ = oracle.mpi(host(A[idx]), host(V0), 10, half=half)
    assert np.max(np.abs(host(s)[idx] - s_ref) / s_ref) < tol
    s32 = s_ref.astype(np.float32)
    s[idx] = torch.from_numpy(s32).to(DEV)
    return s, s32.astype(np.float64)


def test_full_ndb_fp32(stack):
    A, V0 = stack
    idx = SAMPLE + ORACLE_SAMPLE
    s, s_h = pinned_scale(A, V0, dash.DASH_FP32, idx, 1e-5)
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, device=DEV)
    dash.dash_inverse_root_ndb(A, s, N, B, 6, 6, X, status=status, ws=ws)
    del ws
    torch.cuda.empty_cache()
    assert int(status.abs().sum()) == 0
    A_h = host(A[idx])
    X_h = host(X[idx])
    assert np.max(residual(X_h, A_h)) < R_FP32
    k = len(SAMPLE)
    X_ref, _, _ = oracle.ndb_inverse_root(A_h[k:], s_h[k:], 6, 6)
    assert np.max(rel_err(X_h[k:], X_ref)) < ITERATE_TOL
    assert residual_all(X, A) < R_FP32
    del X
    torch.cuda.empty_cache()


def test_full_cn_fp16(stack):
    A, V0 = stack
    s = scale(A, V0, dash.DASH_FP16)
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CN, N, B, dash.DASH_FP16, device=DEV)
    dash.dash_inverse_root_cn(A, s, N, B, 4, 5, dash.DASH_FP16, X, status=status, ws=ws)
    del ws
    torch.cuda.empty_cache()
    assert int(status.abs().sum()) == 0
    idx = SAMPLE + ORACLE_SAMPLE
    A_h = host(A[idx])
    s_h = host(s)[idx]
    s_ref, _ = oracle.mpi(A_h, host(V0), 10, half=True)
    assert np.max(np.abs(s_h - s_ref) / s_ref) < 2e-3
    assert np.max(residual(host(X[idx]), A_h)) < R_FP16
    assert residual_all(X, A) < R_FP16
    del X
    torch.cuda.empty_cache()


def test_full_ndb_half_refine1(stack):
    """Binary16 NDB (6 + 6 steps) with one guarded fp32 correction step, as the bench's solver entry:
    the binary16 storage model on sampled blocks (tolerance 2e-3, fp32 accumulation against exact
    products) and the fp32 residual gate on every block."""
    A, V0 = stack
    idx = SAMPLE + ORACLE_SAMPLE
    s, s_h = pinned_scale(A, V0, dash.DASH_FP32, idx, 1e-5)
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, dash.DASH_FP16, device=DEV)
    dash.dash_inverse_root_ndb_half(A, s, N, B, 6, 6, 1, X, status=status, ws=ws)
    del ws
    torch.cuda.empty_cache()
    assert int(status.abs().sum()) == 0
    A_h = host(A[idx])
    X_h = host(X[idx])
    assert np.max(residual(X_h, A_h)) < R_FP32
    k = len(SAMPLE)
    X_ref = oracle.ndb_half_inverse_root(A_h[k:], s_h[k:], 6, 6, 1)
    assert np.max(rel_err(X_h[k:], X_ref)) < 2e-3
    assert residual_all(X, A) < R_FP32
    del X
    torch.cuda.empty_cache()


def test_full_cn_bf16(stack):
    """CN (5 steps) with bfloat16 iterates after the fp32 scale: the bfloat16 storage model on sampled
    blocks and the bfloat16 residual gate 4e-2 (the binary16 gate scaled by the 8x unit roundoff) on
    every block."""
    A, V0 = stack
    idx = SAMPLE + ORACLE_SAMPLE
    s, s_h = pinned_scale(A, V0, dash.DASH_FP32, idx, 1e-5)
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CN, N, B, dash.DASH_BF16, device=DEV)
    dash.dash_inverse_root_cn(A, s, N, B, 4, 5, dash.DASH_BF16, X, status=status, ws=ws)
    del ws
    torch.cuda.empty_cache()
    assert int(status.abs().sum()) == 0
    A_h = host(A[idx])
    X_h = host(X[idx])
    r_bf16 = 8 * R_FP16
    assert np.max(residual(X_h, A_h)) < r_bf16
    assert np.array_equal(X_h, np.swapaxes(X_h, 1, 2))
    k = len(SAMPLE)
    X_ref, _ = oracle.cn_inverse_root(A_h[k:], s_h[k:], 5, storage="bfloat16")
    assert np.max(rel_err(X_h[k:], X_ref)) < 8 * 5e-3
    assert residual_all(X, A) < r_bf16
    del X
    torch.cuda.empty_cache()


def test_full_step_chebyshev(stack):
    """stack -> EMA stats -> power scale -> Chebyshev d=24 -> apply -> unstack on the full workload."""
    A0, V0 = stack
    A = A0.clone()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(di.SEED_GRADS)
    grads = [torch.randn(sh, generator=gen, device=DEV) * 1e-3 for sh in SHAPES]
    G = torch.empty((NG, B, B), device=DEV)
    dash.dash_stack(grads, B, G)
    # stacking: tile (tr, tc) of weight w sits at offset(w) + tr * cols/B + tc
    assert torch.equal(G[0], grads[0][:B, :B]) and torch.equal(G[NG - 1], grads[-1][B:, -B:])
    sample_t = [0, 700, NG - 1]
    L_prev, R_prev = host(A[sample_t]), host(A[[NG + t for t in sample_t]])
    dash.dash_update_stats(G, NG, B, 0.95, A)
    L_ref, R_ref = oracle.update_stats(host(G[sample_t]), 0.95, L_prev, R_prev)
    assert np.max(rel_err(host(A[sample_t]), L_ref)) < 1e-5
    assert np.max(rel_err(host(A[[NG + t for t in sample_t]]), R_ref)) < 1e-5
    idx = ORACLE_SAMPLE
    s, s_h = pinned_scale(A, V0, dash.DASH_FP32, idx, 1e-5)
    lo = 0.95e-6 / float(s_h.max())  # the damping after one update over the sampled blocks' scale
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, device=DEV)
    dash.dash_inverse_root_cheb(A, s, N, B, 24, lo, 1.25, X, status=status, ws=ws)
    del ws
    assert int(status.abs().sum()) == 0
    X_ref = oracle.cheb_inverse_root(host(A[idx]), s_h, 24, lo, 1.25)
    assert np.max(rel_err(host(X[idx]), X_ref)) < ITERATE_TOL
    # the same solve with split products (fp32 on the bfloat16 matrix cores), same gate
    Xs = torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, dash.DASH_FP32_SPLIT, device=DEV)
    dash.dash_inverse_root_cheb_prec(A, s, N, B, 24, lo, 1.25, dash.DASH_FP32_SPLIT, Xs, status=status, ws=ws)
    del ws
    assert int(status.abs().sum()) == 0
    assert np.max(rel_err(host(Xs[idx]), X_ref)) < ITERATE_TOL
    assert torch.equal(Xs[idx], Xs[idx].transpose(1, 2))
    # and with two-piece binary16 products, same gate
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, dash.DASH_FP32_SPLIT16, device=DEV)
    dash.dash_inverse_root_cheb_prec(A, s, N, B, 24, lo, 1.25, dash.DASH_FP32_SPLIT16, Xs, status=status, ws=ws)
    del ws
    assert int(status.abs().sum()) == 0
    assert np.max(rel_err(host(Xs[idx]), X_ref)) < ITERATE_TOL
    assert torch.equal(Xs[idx], Xs[idx].transpose(1, 2))
    del Xs
    U = torch.empty((NG, B, B), device=DEV)
    ws = dash.workspace(dash.DASH_OP_APPLY, NG, B, device=DEV)
    dash.dash_apply(X[:NG], X[NG:], G, NG, B, U, ws)
    del ws
    t = [3, NG - 2]
    U_ref = oracle.apply(host(X[t]), host(G[t]), host(X[[NG + i for i in t]]))
    assert np.max(rel_err(host(U[t]), U_ref)) < 1e-5
    outs = [torch.empty(sh, device=DEV) for sh in SHAPES]
    dash.dash_unstack(U, B, outs)
    assert torch.equal(outs[0][:B, :B], U[0]) and torch.equal(outs[-1][B:, -B:], U[NG - 1])
    del A, X, U, G, grads, outs
    torch.cuda.empty_cache()


def test_full_step_bench_sequence(stack):
    """The step bench.py times, over two EMA steps with fresh gradients: stack -> statistics
    (two-piece binary16 products) -> power scale (split products) -> Chebyshev d=24 on every block's
    own interval [floor_t / s_i, 1.25] (floor_t = 1e-6 * 0.95^t, the damping after t updates;
    two-piece binary16 products) -> apply (two-piece binary16 products).
    Sampled L and R blocks of one tile are recomputed by the oracle from the same starting blocks and
    gradient tiles through both steps (its own statistics, scale, interval and solve); every sampled
    block's spectrum (numpy eigvalsh; the oracle's Jacobi needs minutes at B = 1024 and is pinned to
    it) lies in its interval."""
    A0, V0 = stack
    A = A0.clone()
    split = dash.DASH_FP32_SPLIT
    cheb_prec = dash.DASH_FP32_SPLIT16
    t_idx = 700
    idx = [t_idx, NG + t_idx]
    L_ref, R_ref = host(A[t_idx]), host(A[NG + t_idx])
    V0h = host(V0)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(di.SEED_GRADS + 1)
    flat = torch.empty(sum(r * c for r, c in SHAPES), device=DEV)
    grads, o = [], 0
    for r, c in SHAPES:
        grads.append(flat[o:o + r * c].view(r, c))
        o += r * c
    G = torch.empty((NG, B, B), device=DEV)
    U = torch.empty((NG, B, B), device=DEV)
    X = torch.empty_like(A)
    s = torch.empty(N, device=DEV)
    lo = torch.empty(N, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws_s = dash.workspace(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 32, device=DEV)
    ws_c = dash.workspace(dash.DASH_OP_CHEB, N, B, cheb_prec, device=DEV)
    ws_a = dash.workspace(dash.DASH_OP_APPLY, NG, B, device=DEV)
    ws_st = dash.workspace(dash.DASH_OP_STATS, NG, B, cheb_prec, device=DEV)
    floor = 1e-6
    for step in range(2):
        flat.normal_(0.0, 1e-3, generator=gen)
        floor *= 0.95
        dash.dash_stack(grads, B, G)
        dash.dash_update_stats_ws(G, NG, B, 0.95, cheb_prec, A, ws_st)
        dash.dash_scale(A, N, B, dash.DASH_SCALE_POWER, split, 32, 10, V0, s, ws_s)
        dash.dash_inverse_root_cheb_blocks(A, s, N, B, 24, floor, None, 1.0, 1.25, cheb_prec, X, lo_out=lo,
                                          status=status, ws=ws_c)
        dash.dash_apply_prec(X[:NG], X[NG:], G, NG, B, cheb_prec, U, ws_a)
        # the oracle's copy of the same step for tile t_idx, from the gradient itself
        G_t = tile_of(grads, t_idx)
        L_ref, R_ref = oracle.update_stats(G_t, 0.95, L_ref, R_ref)
    assert int(status.abs().sum()) == 0
    A_ref = np.stack([L_ref, R_ref])
    assert np.max(rel_err(host(A[idx]), A_ref)) < 1e-5
    s_ref, _ = oracle.mpi(A_ref, V0h, 10)
    assert np.max(np.abs(host(s[idx]) - s_ref) / s_ref) < 1e-5
    lo_ref = oracle.cheb_interval_lo(s_ref, floor)
    assert np.max(np.abs(host(lo[idx]) - lo_ref) / lo_ref) < 1e-5
    for b in range(2):
        w = np.linalg.eigvalsh(A_ref[b])
        assert lo_ref[b] * s_ref[b] <= w[0] and w[-1] <= 1.25 * s_ref[b], (b, w[0], w[-1], s_ref[b])
    X_ref = oracle.cheb_inverse_root(A_ref, s_ref, 24, lo_ref, 1.25)
    assert np.max(rel_err(host(X[idx]), X_ref)) < ITERATE_TOL
    U_ref = oracle.apply(X_ref[0], G_t, X_ref[1])
    assert np.max(rel_err(host(U[t_idx]), U_ref)) < ITERATE_TOL
    del A, X, U, G, flat, grads, ws_s, ws_c, ws_a, ws_st
    torch.cuda.empty_cache()


@pytest.mark.parametrize("prec,refine", [(dash.DASH_FP32, 0), (dash.DASH_FP16, 1)])
def test_full_evd(stack, prec, refine):
    """The block-Jacobi eigendecomposition on the full stack, in fp32 and with the binary16 first
    pass (then the fp32 refinement pass).  The fp64 oracle needs minutes per 1024-block, so here the
    checks are properties of every block: it converged (status 0), its eigenvalues keep the block's
    trace and Frobenius norm (sum w = tr A, sum w^2 = ||A||_F^2, evaluated in fp64), the residual
    holds at the fp32 gate, and X is exactly symmetric."""
    A, _ = stack
    X = torch.empty_like(A)
    w = torch.empty((N, B), device=DEV)
    sweeps = torch.empty(N, dtype=torch.int32, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_EVD, N, B, device=DEV)
    dash.dash_inverse_root_evd_prec(A, N, B, 20, refine, prec, X, eigvals=w, sweeps=sweeps, status=status, ws=ws)
    del ws
    torch.cuda.empty_cache()
    assert int(status.abs().sum()) == 0
    assert int(sweeps.max()) < 20 * (1 + refine)
    for i in range(0, N, 256):
        a = A[i:i + 256].double()
        wd = w[i:i + 256].double()
        tr = torch.diagonal(a, dim1=1, dim2=2).sum(1)
        fro2 = (a * a).sum((1, 2))
        assert float(((wd.sum(1) - tr).abs() / tr).max()) < 1e-5
        assert float((((wd * wd).sum(1) - fro2).abs() / fro2).max()) < 1e-5
        del a
    X_h = host(X[SAMPLE])
    assert np.max(residual(X_h, host(A[SAMPLE]))) < R_FP32
    assert np.array_equal(X_h, np.swapaxes(X_h, 1, 2))
    assert residual_all(X, A) < R_FP32
    del X, w
    torch.cuda.empty_cache()
