"""GPU parity of the bfloat16-operand solvers (DASH_BF16): Coupled Newton p=4 (dash_inverse_root_cn)
and NDB with bfloat16 iterates and the guarded fp32 correction (dash_inverse_root_ndb_lowp), against
the oracle's bfloat16-storage models of the same algorithms (every stored iterate rounded to
bfloat16, exact products; pinned on the CPU by the scalar recurrences on diagonal blocks).

Gates: bfloat16 keeps 8 significant bits where binary16 keeps 11, so its unit roundoff 2^-8 is 8x
binary16's 2^-11, and the binary16 gates scale by 8: residual ||X^4 A - I||_F / sqrt(B) <= 4e-2, model
parity (GPU against the storage model, which differ by where fp32 accumulation moves a rounding)
<= 4e-2 for CN and <= 1.6e-2 for NDB.  Scaling is fp32 power iteration (bfloat16 scaling is not
offered: binary16 already streams A at two bytes)."""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import DEV, R_FP16, cn, cn_adaptive, host_power_scale, rel_err, residual, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_RATIO = 8.0  # unit roundoff of bfloat16 over binary16
R_BF16 = BF16_RATIO * R_FP16
CN_TOL = BF16_RATIO * 5e-3
NDB_TOL = BF16_RATIO * 2e-3


def ndb_lowp(A, s, it1, it2, refine, prec=dash.DASH_BF16):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    mon = torch.empty((N, it1 + it2), device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, prec, device=DEV)
    dash.dash_inverse_root_ndb_lowp(A, s, N, B, it1, it2, prec, refine, X, monitor=mon, status=status, ws=ws)
    return X, mon, status


def gram(N, B, seed):
    g = di.rng(seed)
    A = np.empty((N, B, B), dtype=np.float32)
    for i in range(N):
        G = g.standard_normal((B, B)) * 1e-3
        M = G @ G.T / B + 1e-6 * np.eye(B)
        A[i] = (0.5 * (M + M.T)).astype(np.float32)
    return A


@pytest.mark.parametrize("B", [64, 192, 256, 512])
def test_cn_bf16_matches_storage_model(B):
    """kappa 5 stacks; B % 256 == 0 runs the 256-wide triangle kernel, 64 and 192 the 64-wide one."""
    A = di.known_spectrum_stack(300 + B, 3, B, 0.2, 1.0)[0].astype(np.float32)
    Ad = to_dev(A)
    s = host_power_scale(A, di.start_vectors(B, 32))
    X, mon, status = cn(Ad, s, 9, dash.DASH_BF16, want_monitor=True)
    Xh = to_host(X)
    assert np.all(to_host(status) == 0)
    ref, mon_ref = oracle.cn_inverse_root(A, to_host(s), 9, storage="bfloat16")
    err, r = rel_err(Xh, ref), residual(Xh, A)
    print("B", B, "model err", err.max(), "residual", r.max())
    assert err.max() <= CN_TOL
    assert r.max() <= R_BF16
    assert np.array_equal(Xh, Xh.transpose(0, 2, 1))  # triangle-only products, mirrored
    m = to_host(mon)
    assert np.max(np.abs(m[:, :3] - mon_ref[:, :3]) / mon_ref[:, :3]) < 8e-2
    # bfloat16 storage costs accuracy against binary16 storage of the same iteration
    Xf16, _, _ = cn(Ad, s, 9, dash.DASH_FP16)
    assert residual(to_host(Xf16), A).max() < r.max()


def test_cn_bf16_reads_only_the_upper_triangle():
    A = di.known_spectrum_stack(330, 2, 256, 0.2, 1.0)[0].astype(np.float32)
    noisy = A.copy()
    low = np.tril_indices(256, -1)
    noisy[:, low[0], low[1]] += di.gaussian((2, len(low[0])), 331, 0.05)
    s = torch.ones(2, device=DEV)
    X_clean, _, _ = cn(to_dev(A), s, 6, dash.DASH_BF16)
    X_noisy, _, _ = cn(to_dev(noisy), s, 6, dash.DASH_BF16)
    assert torch.equal(X_clean, X_noisy)


@pytest.mark.parametrize("name", ["tiny", "gram256"])
def test_ndb_bf16_matches_storage_model(name):
    """bfloat16 NDB against its storage model; at kappa ~5 every guarded correction step is taken
    and lowers the residual, the first by at least half (the rounding noise that does not commute
    with A is removed only linearly: binary16 NDB shows the same 2-3x per step)."""
    A = di.tiny_stack() if name == "tiny" else gram(4, 256, 93)
    s = (np.linalg.eigvalsh(A.astype(np.float64))[:, -1] * 1.02).astype(np.float32)
    Ad, sd = to_dev(A), to_dev(s)
    r_prev = None
    for refine in range(3):
        X, mon, status = ndb_lowp(Ad, sd, 6, 6, refine)
        assert (to_host(status) == 0).all()
        Xh = to_host(X)
        ref = oracle.ndb_half_inverse_root(A.astype(np.float64), s.astype(np.float64), 6, 6, refine,
                                           storage="bfloat16")
        err, r = rel_err(Xh, ref), residual(Xh, A)
        print(name, "refine", refine, "model err", err.max(), "residual", r.max())
        assert err.max() <= NDB_TOL
        if refine == 0:
            assert r.max() <= R_BF16
        elif name == "gram256":
            assert np.all(r < r_prev)
            assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))
            if refine == 1:
                assert np.all(r <= r_prev / 2)
        else:  # the guard never lets a step raise the residual
            assert np.all(r <= r_prev * (1 + 1e-6))
        r_prev = r


def test_ndb_lowp_binary16_is_ndb_half():
    """dash_inverse_root_ndb_lowp with DASH_FP16 is dash_inverse_root_ndb_half, bit for bit."""
    A = gram(2, 128, 94)
    s = to_dev((np.linalg.eigvalsh(A.astype(np.float64))[:, -1] * 1.02).astype(np.float32))
    Ad = to_dev(A)
    X1, _, _ = ndb_lowp(Ad, s, 5, 5, 1, dash.DASH_FP16)
    X2 = torch.empty_like(Ad)
    ws = dash.workspace(dash.DASH_OP_NDB, 2, 128, dash.DASH_FP16, device=DEV)
    dash.dash_inverse_root_ndb_half(Ad, s, 2, 128, 5, 5, 1, X2, ws=ws)
    assert torch.equal(X1, X2)


def test_cn_adaptive_bf16():
    """Per-block stopping with bfloat16 iterates: each block's result equals the fixed bfloat16 run
    of its length up to the one rounding of the stored X_k."""
    lam_min = [0.5, 1e-1, 1e-2]
    A = np.concatenate([di.known_spectrum_stack(340 + i, 1, 256, lm, 1.0)[0] for i, lm in enumerate(lam_min)])
    A = A.astype(np.float32)
    s = np.ones(len(A), dtype=np.float32)
    T, tol = 20, 5e-2
    X, mon, steps, status = cn_adaptive(to_dev(A), to_dev(s), T, tol, dash.DASH_BF16)
    assert (to_host(status) == 0).all()
    mon, steps, X = to_host(mon), to_host(steps).astype(int), to_host(X)
    for b in range(len(A)):
        k = steps[b]
        assert 1 <= k <= T and np.all(mon[b, 1:k] > tol) and (k == T or mon[b, k] <= tol)
        Xf, _, _ = cn(to_dev(A[b:b + 1]), to_dev(s[b:b + 1]), int(k), dash.DASH_BF16)
        assert rel_err(X[b], to_host(Xf)[0])[0] <= BF16_RATIO * 2e-3
    assert steps[0] < steps[-1]
