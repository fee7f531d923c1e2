"""GPU parity of the per-block Chebyshev interval, the smallest-eigenvalue estimate, the residual probe
and the routed (per-block solver choice) inverse root, against the CPU oracle.

Every scale s fed to the GPU and to the oracle here is the oracle's own power-iteration estimate
rounded to fp32, and every X handed to the probe is built on the host, so no oracle input comes from
the GPU path.  Gates: fp32 iterate parity 1e-4; residual ||X^4 A - I||_F / sqrt(B) <= 1e-3 in fp64 on
the host.
"""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import DEV, ITERATE_TOL, R_FP32, rel_err, residual, to_dev, to_host

pytestmark = pytest.mark.gpu

HI = 1.25


def mixed_stack(seed, n_each, B, spans):
    """Blocks of known spectra: n_each blocks per (lam_min, lam_max) span, each scaled by its own
    power of ten so that the blocks' scales differ."""
    As, Qs, lams = [], [], []
    for q, (lo, hi) in enumerate(spans):
        A, Q, lam = di.known_spectrum_stack(seed + q, n_each, B, lo, hi)
        f = 10.0 ** (-q - 3)
        As.append(A * f)
        Qs.append(Q)
        lams.append(lam * f)
    return np.concatenate(As).astype(np.float32), np.concatenate(Qs), np.concatenate(lams)


def oracle_scale(A, V0, steps=10):
    """The oracle's power-iteration scale, rounded to fp32 (fed to both sides)."""
    s, _ = oracle.mpi(A.astype(np.float64), V0, steps)
    return np.asarray(s, dtype=np.float32)


def cheb_blocks(Ad, s, degree, floor, lam=None, theta=1.0, prec=dash.DASH_FP32):
    N, B = Ad.shape[0], Ad.shape[1]
    X = torch.empty_like(Ad)
    lo = torch.empty(N, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, prec, device=DEV)
    dash.dash_inverse_root_cheb_blocks(Ad, s, N, B, degree, floor, lam, theta, HI, prec, X, lo_out=lo,
                                      status=status, ws=ws)
    return X, lo, status


@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP32_SPLIT, dash.DASH_FP32_SPLIT16])
@pytest.mark.parametrize("degree", [1, 2, 3, 8, 24])
def test_cheb_blocks_floor_interval_matches_oracle(prec, degree):
    """Each block's interval [floor / s_i, hi] is derived on the device; blocks of different scales
    and conditioning get different intervals, each as the oracle computes it."""
    A, _, lam = mixed_stack(200, 2, 256, [(0.05, 1.0), (1e-3, 1.0), (0.3, 1.0)])
    V0 = di.start_vectors(256, 32)
    s = oracle_scale(A, V0)
    floor = 0.9 * float(lam.min())
    X, lo, status = cheb_blocks(to_dev(A), to_dev(s), degree, floor, prec=prec)
    lo_ref = oracle.cheb_interval_lo(s.astype(np.float64), floor)
    assert np.array_equal(to_host(lo), lo_ref.astype(np.float32).astype(np.float64))
    assert np.all(to_host(lo) * s <= lam.min(axis=1))                # the interval holds every spectrum
    X_ref = oracle.cheb_inverse_root(A, s.astype(np.float64), degree, lo_ref, HI)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    assert np.all(to_host(status) == 0)


def test_cheb_blocks_estimate_and_shared_interval_bitwise():
    """With per-block estimates the lower end is max(floor, theta lam_i) / s_i; with every s_i = 1 and
    no estimate the call is bit for bit the shared-interval call on [floor, hi]."""
    A, _, lam = mixed_stack(210, 2, 256, [(0.1, 1.0), (0.02, 1.0)])
    V0 = di.start_vectors(256, 32)
    s = oracle_scale(A, V0)
    est = (lam.min(axis=1) * np.array([3.0, 1.0, 1.5, 0.5])).astype(np.float32)
    floor = 0.5 * float(lam.min())
    X, lo, status = cheb_blocks(to_dev(A), to_dev(s), 16, floor, lam=to_dev(est), theta=0.5,
                                prec=dash.DASH_FP32_SPLIT)
    lo_ref = oracle.cheb_interval_lo(s.astype(np.float64), floor, lam=est.astype(np.float64), theta=0.5)
    assert np.array_equal(to_host(lo), lo_ref.astype(np.float32).astype(np.float64))
    X_ref = oracle.cheb_inverse_root(A, s.astype(np.float64), 16, lo_ref, HI)
    assert np.max(rel_err(to_host(X), X_ref)) < ITERATE_TOL
    Ad = to_dev(A / s[:, None, None])
    ones = torch.ones(4, device=DEV)
    Xb, _, _ = cheb_blocks(Ad, ones, 16, 0.03, prec=dash.DASH_FP32_SPLIT)
    Xs = torch.empty_like(Ad)
    ws = dash.workspace(dash.DASH_OP_CHEB, 4, 256, dash.DASH_FP32_SPLIT, device=DEV)
    dash.dash_inverse_root_cheb_prec(Ad, ones, 4, 256, 16, 0.03, HI, dash.DASH_FP32_SPLIT, Xs, ws=ws)
    assert torch.equal(Xb, Xs)


def test_cheb_blocks_bad_interval_is_flagged_and_isolated():
    """A block whose lower end reaches hi (its scale far below the floor) is flagged (status bit 0) and
    written NaN; the other blocks are unaffected."""
    A, _, lam = mixed_stack(220, 2, 128, [(0.1, 1.0)])
    s = np.array([1.0, 1e-3], dtype=np.float32)
    X, lo, status = cheb_blocks(to_dev(A), to_dev(s), 8, 0.05)
    st = to_host(status)
    assert st[0] == 0 and (int(st[1]) & 1) == 1
    assert bool(torch.isnan(X[1]).all()) and np.isnan(to_host(lo)[1])
    X_ref = oracle.cheb_inverse_root(A[:1], 1.0, 8, 0.05, HI)
    assert np.max(rel_err(to_host(X[:1]), X_ref)) < ITERATE_TOL


def test_spectrum_min_matches_oracle():
    A, _, lam = mixed_stack(230, 2, 256, [(0.05, 1.0), (1e-3, 1.0)])
    N, B = A.shape[0], A.shape[1]
    V0 = di.start_vectors(B, 32)
    s = oracle_scale(A, V0)
    lam_d = torch.empty(N, device=DEV)
    ws = dash.workspace(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 32, device=DEV)
    for steps in (1, 10, 40):
        dash.dash_spectrum_min(to_dev(A), to_dev(s), N, B, HI, 32, steps, to_dev(V0), lam_d, ws)
        ref, _ = oracle.mpi_shifted(A.astype(np.float64), HI * s.astype(np.float64), V0, steps)
        got = to_host(lam_d)
        # lam = sigma - mu: compare on the scale of sigma (the cancellation leaves fp32 rounding of sigma)
        assert np.max(np.abs(got - ref) / (HI * s)) < 1e-5, steps
        assert np.all(got >= lam.min(axis=1) - 1e-5 * HI * s)


def test_residual_probe_matches_oracle():
    """The probe on host-built roots: exact (closed form) and perturbed ones."""
    A64, Q, lam = di.known_spectrum_stack(240, 4, 256, 0.01, 1.0)
    X = np.einsum("bij,bj,bkj->bik", Q, lam ** -0.25, Q)
    g = di.rng(241)
    X[1:] += np.array([1e-4, 1e-3, 1e-2])[:, None, None] * g.standard_normal((3, 256, 256)) / 16
    A, X = A64.astype(np.float32), X.astype(np.float32)
    V0 = di.start_vectors(256, 32)
    r = torch.empty(4, device=DEV)
    ws = dash.workspace(dash.DASH_OP_SCALE, 4, 256, dash.DASH_FP32, 32, device=DEV)
    dash.dash_residual_probe(to_dev(A), to_dev(X), 4, 256, 32, to_dev(V0), r, ws)
    ref = oracle.residual_probe(A, X, V0)
    got = to_host(r)
    assert np.all(np.abs(got - ref) <= 1e-3 * ref + 2e-5), (got, ref)
    # the probe tracks the gate's residual (32 probes: within a factor of two here)
    exact = residual(X, A)
    assert np.all(got[1:] > 0.5 * exact[1:]) and np.all(got[1:] < 2.0 * exact[1:])


@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP32_SPLIT, dash.DASH_FP32_SPLIT16])
def test_routed_inverse_root_matches_oracle(prec):
    """Blocks of kappa ~ 4 stay with Chebyshev on their estimated intervals; kappa 1e4 blocks go to
    coupled Newton.  Routes equal the oracle's, roots meet the iterate-parity and residual gates."""
    A, _, lam = mixed_stack(250, 3, 256, [(0.25, 1.0), (1e-4, 1.0)])
    N, B = A.shape[0], A.shape[1]
    V0 = di.start_vectors(B, 32)
    s = oracle_scale(A, V0)
    floor = 0.9 * float(lam.min())
    tol, degree, est, cn_iters = 1e-3, 16, 10, 30
    X = torch.empty((N, B, B), device=DEV)
    lam_d, resid = torch.empty(N, device=DEV), torch.empty(N, device=DEV)
    route = torch.empty(N, dtype=torch.int32, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_ROUTED, N, B, device=DEV)
    dash.dash_inverse_root_routed(to_dev(A), to_dev(s), N, B, degree, floor, HI, 32, est, to_dev(V0), tol,
                                  cn_iters, prec, X, lam_min=lam_d, resid=resid, route=route, status=status,
                                  ws=ws)
    X_ref, route_ref, lam_ref, r_ref = oracle.routed_inverse_root(A, s.astype(np.float64), degree, floor, HI, V0,
                                                                  est, tol, cn_iters)
    assert list(to_host(route).astype(int)) == list(route_ref) == [0, 0, 0, 1, 1, 1]
    assert np.max(np.abs(to_host(lam_d) - lam_ref) / (HI * s)) < 1e-5
    Xh = to_host(X)
    assert np.max(rel_err(Xh, X_ref)) < ITERATE_TOL
    assert np.max(residual(Xh, A)) < R_FP32
    assert np.all(to_host(status) == 0)
    rh = to_host(resid)
    assert np.all(rh < tol)


def test_seeded_start_pool_equals_the_host_pool():
    """dash_scale without start vectors draws the pool on the device from the seed: the pool is the
    host twin's bit for bit, and the scale equals the one computed from the host pool."""
    Vd = torch.empty((256, 32), device=DEV)
    dash.dash_start_vectors(256, 32, 7, Vd)
    V0 = di.start_pool_counter(256, 32, 7)
    assert np.array_equal(to_host(Vd), V0.astype(np.float64))
    A, _, _ = mixed_stack(260, 2, 256, [(0.05, 1.0), (1e-3, 1.0)])
    N, B = A.shape[0], A.shape[1]
    Ad = to_dev(A)
    ws = dash.workspace(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 32, device=DEV)
    s_seed, s_pool, s_na = (torch.empty(N, device=DEV) for _ in range(3))
    dash.dash_scale(Ad, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, None, s_seed, ws, seed=7)
    dash.dash_scale(Ad, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, to_dev(V0), s_pool, ws)
    dash.dash_scale_noalloc(Ad, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, None, s_na, seed=7)
    assert torch.equal(s_seed, s_pool) and torch.equal(s_seed, s_na)
    s_ref, _ = oracle.mpi(A.astype(np.float64), V0, 10)
    assert np.max(np.abs(to_host(s_seed) - s_ref) / s_ref) < 1e-5


def test_binding_rejects_bad_tensor_arguments():
    """Wrong dtype, too few elements, a non-contiguous view: refused by the binding before any pointer
    reaches the library."""
    A = torch.eye(64, device=DEV).repeat(2, 1, 1)
    s = torch.ones(2, device=DEV)
    X = torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_NDB, 2, 64, device=DEV)
    with pytest.raises(ValueError, match="float32"):
        dash.dash_inverse_root_ndb(A.double(), s, 2, 64, 3, 3, X, ws=ws)
    with pytest.raises(ValueError, match="elements"):
        dash.dash_inverse_root_ndb(A[:1], s, 2, 64, 3, 3, X, ws=ws)
    with pytest.raises(ValueError, match="contiguous"):
        dash.dash_inverse_root_ndb(A.transpose(1, 2), s, 2, 64, 3, 3, X, ws=ws)
    with pytest.raises(ValueError, match="int32"):
        dash.dash_inverse_root_ndb(A, s, 2, 64, 3, 3, X, status=torch.zeros(2, device=DEV), ws=ws)
    with pytest.raises(ValueError, match="unit column stride"):
        dash.dash_stack([torch.zeros((128, 128), device=DEV).t()[::1, ::2]], 64, torch.empty((2, 64, 64), device=DEV))
