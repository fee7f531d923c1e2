"""GPU parity of the 1-D parameter path (pieces of B, rank-one statistics, inverse square root by one
NDB call, block-times-vector apply) against the CPU oracle.  Scales fed to both sides are the oracle's
own power-iteration estimates rounded to fp32."""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import DEV, ITERATE_TOL, R_FP32, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def pieces_of(lens, B):
    return sum(-(-n // B) for n in lens)


def test_vec_stack_round_trip_and_padding():
    B = 64
    lens = [5, 64, 130, 1, 1000]
    vs = [to_dev(di.gaussian((n,), 90 + i)) for i, n in enumerate(lens)]
    P = pieces_of(lens, B)
    g = torch.full((P, B), 7.0, device=DEV)
    dash.dash_stack_vec(vs, B, g)
    ref = oracle.stack_vec([to_host(v) for v in vs], B)
    assert np.array_equal(to_host(g), ref)
    outs = [torch.full((n,), -1.0, device=DEV) for n in lens]
    dash.dash_unstack_vec(g, B, outs)
    assert all(torch.equal(a, b) for a, b in zip(outs, vs))


@pytest.mark.parametrize("B", [64, 256, 1024])
def test_vec_stats_and_apply(B):
    P = 3
    g = di.rng(91 + B)
    gi = g.integers(-8, 9, (P, B)).astype(np.float32)
    L0 = g.integers(-8, 9, (P, B, B)).astype(np.float32)
    L0 = L0 + np.swapaxes(L0, 1, 2)
    L = to_dev(L0)
    dash.dash_update_stats_vec(to_dev(gi), P, B, 0.5, L)
    Lh = to_host(L)
    assert np.array_equal(Lh, oracle.update_stats_vec(gi, 0.5, L0))          # exact on small integers
    assert np.array_equal(Lh, np.swapaxes(Lh, 1, 2))
    gg = di.gaussian((P, B), 92 + B)
    Lg0 = np.stack([np.eye(B, dtype=np.float32)] * P) * 1e-3
    Lg = to_dev(Lg0)
    dash.dash_update_stats_vec(to_dev(gg), P, B, 0.95, Lg)
    assert np.max(rel_err(to_host(Lg), oracle.update_stats_vec(gg, 0.95, Lg0))) < 1e-6
    X = di.gaussian((P, B, B), 93 + B)
    u = torch.empty((P, B), device=DEV)
    dash.dash_apply_vec(to_dev(X), to_dev(gg), P, B, u)
    u_ref = oracle.apply_vec(X, gg)
    assert np.max(np.abs(to_host(u) - u_ref) / np.linalg.norm(u_ref, axis=1, keepdims=True)) < 1e-6
    dash.dash_apply_vec(to_dev(np.stack([np.eye(B, dtype=np.float32)] * P)), to_dev(gg), P, B, u)
    assert np.array_equal(to_host(u), gg.astype(np.float64))


@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP32_SPLIT])
@pytest.mark.parametrize("iters", [1, 2, 6, 14])
def test_inverse_sqrt_ndb_matches_oracle(prec, iters):
    A64, Q, lam = di.known_spectrum_stack(94, 4, 256, 1e-2, 1.0)
    A = A64.astype(np.float32)
    s = (lam.max(axis=1) * 1.01).astype(np.float32)
    X = torch.empty((4, 256, 256), device=DEV)
    status = torch.empty(4, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, 4, 256, prec, device=DEV)
    dash.dash_inverse_sqrt_ndb(to_dev(A), to_dev(s), 4, 256, iters, prec, X, status=status, ws=ws)
    X_ref = oracle.ndb_inverse_sqrt(A, s.astype(np.float64), iters)
    Xh = to_host(X)
    assert np.max(rel_err(Xh, X_ref)) < ITERATE_TOL
    assert np.all(to_host(status) == 0)
    if iters == 14:  # converged: X^2 A = I
        r = np.linalg.norm(Xh @ Xh @ A.astype(np.float64) - np.eye(256), axis=(1, 2)) / 16
        assert np.max(r) < R_FP32


def test_vec_step_matches_oracle():
    """The optimizer step of 1-D parameters: the Llama model's norm gains (49 vectors of 2048) and two
    ragged vectors, B = 1024: pieces -> statistics (prior eps I) -> power scale -> inverse square root
    (NDB, 14 steps) -> apply -> vectors.  Two pieces recomputed by the oracle from the same start."""
    B, eps, beta = 1024, 1e-6, 0.95
    lens = [2048] * 49 + [1000, 3000]
    P = pieces_of(lens, B)
    vs = [to_dev(di.gaussian((n,), 95 + i, std=1e-3)) for i, n in enumerate(lens)]
    g = torch.empty((P, B), device=DEV)
    dash.dash_stack_vec(vs, B, g)
    L = (torch.eye(B, device=DEV) * eps).repeat(P, 1, 1)
    dash.dash_update_stats_vec(g, P, B, beta, L)
    V0 = torch.from_numpy(di.start_vectors(B, 32)).to(DEV)
    s = torch.empty(P, device=DEV)
    ws = dash.workspace(dash.DASH_OP_SCALE, P, B, dash.DASH_FP32, 32, device=DEV)
    dash.dash_scale(L, P, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, V0, s, ws)
    X = torch.empty_like(L)
    ws = dash.workspace(dash.DASH_OP_NDB, P, B, dash.DASH_FP32_SPLIT, device=DEV)
    status = torch.empty(P, dtype=torch.int32, device=DEV)
    dash.dash_inverse_sqrt_ndb(L, s, P, B, 14, dash.DASH_FP32_SPLIT, X, status=status, ws=ws)
    u = torch.empty((P, B), device=DEV)
    dash.dash_apply_vec(X, g, P, B, u)
    outs = [torch.empty(n, device=DEV) for n in lens]
    dash.dash_unstack_vec(u, B, outs)
    assert int(status.abs().sum()) == 0
    idx = [3, P - 1]  # a norm-gain piece, and the last piece of the ragged 3000 (zero-padded)
    g_ref = oracle.stack_vec([to_host(v) for v in vs], B)[idx]
    L_ref = oracle.update_stats_vec(g_ref, beta, np.stack([np.eye(B) * eps] * 2))
    s_ref, _ = oracle.mpi(L_ref, di.start_vectors(B, 32), 10)
    X_ref = oracle.ndb_inverse_sqrt(L_ref, s_ref, 14)
    assert np.max(rel_err(to_host(X[idx]), X_ref)) < ITERATE_TOL
    u_ref = oracle.apply_vec(X_ref, g_ref)
    assert np.max(rel_err(to_host(u[idx])[:, None, :], u_ref[:, None, :])) < ITERATE_TOL
    back = oracle.unstack_vec(to_host(u), lens, B)
    assert all(np.array_equal(to_host(o), b) for o, b in zip(outs, back))
