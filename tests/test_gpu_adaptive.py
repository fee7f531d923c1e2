"""GPU parity of the per-block adaptive NDB and Coupled-Newton calls (each block stops before a step
k >= 1 once its monitor is <= tol) on a stack whose blocks need different step counts
(condition numbers 2 .. 1e4).

Checked per block: the GPU's decision follows the rule on its own monitors (every monitor before the
stop is > tol, the one at the stop is <= tol, nothing is computed after it); the result equals the
oracle's fixed-step run of the same lengths (iterate parity 1e-4); and the step counts equal the
oracle's adaptive decision wherever the oracle's monitors are clear of tol by a factor 2 (near tol,
fp32 and fp64 monitors may decide a step apart, and both decisions are valid).
"""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import (DEV, ITERATE_TOL, R_FP32, cn, cn_adaptive, ndb, ndb_adaptive, rel_err, residual, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu

B = 128
LAM_MIN = [0.5, 1e-1, 1e-2, 1e-3, 1e-4]


@pytest.fixture(scope="module")
def mixed():
    A = np.concatenate([di.known_spectrum_stack(100 + i, 1, B, lm, 1.0)[0] for i, lm in enumerate(LAM_MIN)])
    A = A.astype(np.float32)
    return A, np.ones(len(LAM_MIN), dtype=np.float32)


def check_rule(mon, k, tol, T):
    """mon: one call's monitor row on the GPU; k: the steps it reports."""
    assert 1 <= k <= T
    assert np.all(mon[1:k] > tol)
    if k < T:
        assert mon[k] <= tol
        assert np.all(mon[k + 1:T] == 0.0)


def clear(mon, k, tol, T):
    """The oracle's decision at k is clear of tol by a factor 2 on both sides."""
    above = k <= 1 or mon[k - 1] >= 2 * tol
    below = k >= T or mon[k] <= tol / 2
    return above and below


@pytest.mark.parametrize("tol", [1e-5, 1e-3])
def test_ndb_adaptive_mixed_stack(mixed, tol):
    A, s = mixed
    T = 20
    X, mon, steps, status = ndb_adaptive(to_dev(A), to_dev(s), T, T, tol)
    assert (to_host(status) == 0).all()
    mon, steps, X = to_host(mon), to_host(steps).astype(int), to_host(X)
    _, mon_o, st_o = oracle.ndb_inverse_root_adaptive(A, s, T, T, tol)
    for b in range(len(A)):
        check_rule(mon[b, :T], steps[b, 0], tol, T)
        check_rule(mon[b, T:], steps[b, 1], tol, T)
        Xf, _, _ = oracle.ndb_inverse_root(A[b], 1.0, int(steps[b, 0]), int(steps[b, 1]))
        assert rel_err(X[b], Xf)[0] <= ITERATE_TOL
        for c in range(2):
            if clear(mon_o[b, c * T:(c + 1) * T], st_o[b, c], tol, T):
                assert steps[b, c] == st_o[b, c]
    # better-conditioned blocks stop earlier, and no block ran every step
    assert np.all(np.diff(steps[:, 0]) >= 0) and steps[0, 0] < steps[-1, 0]
    assert np.all(steps < T)
    if tol <= 1e-5:
        assert residual(X, A).max() <= R_FP32


def stopped_only_at_exact_fixed_points(mon, steps, T):
    """tol = 0 stops a call only where its monitor is exactly 0: the iterate is then a fixed point
    of the fp32 iteration (S = I exactly), so the later steps would not have changed it."""
    for k in np.atleast_1d(steps):
        assert 1 <= k <= T
        if k < T:
            assert mon[k] == 0.0


def test_ndb_adaptive_zero_tol_is_the_fixed_call(mixed):
    """With tol = 0 the result is the fixed-step call's, bit for bit."""
    A, s = mixed
    Xa, mon, steps, _ = ndb_adaptive(to_dev(A), to_dev(s), 7, 6, 0.0)
    Xf, _, _, _ = ndb(to_dev(A), to_dev(s), 7, 6)
    assert torch.equal(Xa, Xf)
    mon, steps = to_host(mon), to_host(steps).astype(int)
    for b in range(len(A)):
        stopped_only_at_exact_fixed_points(mon[b, :7], steps[b, 0], 7)
        stopped_only_at_exact_fixed_points(mon[b, 7:], steps[b, 1], 6)


@pytest.mark.parametrize("tol", [1e-5, 1e-3])
def test_cn_adaptive_mixed_stack(mixed, tol):
    A, s = mixed
    T = 25
    X, mon, steps, status = cn_adaptive(to_dev(A), to_dev(s), T, tol)
    assert (to_host(status) == 0).all()
    mon, steps, X = to_host(mon), to_host(steps).astype(int), to_host(X)
    _, mon_o, st_o = oracle.cn_inverse_root_adaptive(A, s, T, tol)
    for b in range(len(A)):
        check_rule(mon[b], steps[b], tol, T)
        Xf, _ = oracle.cn_inverse_root(A[b], 1.0, int(steps[b]))
        assert rel_err(X[b], Xf)[0] <= ITERATE_TOL
        if clear(mon_o[b], st_o[b], tol, T):
            assert steps[b] == st_o[b]
    assert np.all(np.diff(steps) >= 0) and steps[0] < steps[-1]
    # the CN monitor is the residual of X_k (in exact arithmetic): stopping at tol bounds it, up to
    # the fp32 floor
    assert np.all(residual(X, A) <= max(2 * tol, R_FP32))


def test_cn_adaptive_zero_tol_is_the_fixed_call(mixed):
    A, s = mixed
    Xa, mon, steps, _ = cn_adaptive(to_dev(A), to_dev(s), 9, 0.0)
    Xf, _, _ = cn(to_dev(A), to_dev(s), 9)
    assert torch.equal(Xa, Xf)
    mon, steps = to_host(mon), to_host(steps).astype(int)
    for b in range(len(A)):
        stopped_only_at_exact_fixed_points(mon[b], steps[b], 9)


@pytest.mark.parametrize("B16", [128, 256])
def test_cn_adaptive_binary16(B16):
    """Binary16 iterates (128- and 256-wide tile kernels): the rule on the GPU's own monitors; each
    block's result equals the fixed binary16 run of its length up to the one binary16 rounding of
    the stored X_k, and (for condition numbers up to 100) the exact fp64 oracle run of its length to
    binary16 accuracy, with the residual at the monitor's level."""
    A = np.concatenate([di.known_spectrum_stack(200 + i, 1, B16, lm, 1.0)[0] for i, lm in enumerate(LAM_MIN)])
    A = A.astype(np.float32)
    s = np.ones(len(A), dtype=np.float32)
    T, tol = 20, 1e-2
    X, mon, steps, status = cn_adaptive(to_dev(A), to_dev(s), T, tol, dash.DASH_FP16)
    assert (to_host(status) == 0).all()
    mon, steps, X = to_host(mon), to_host(steps).astype(int), to_host(X)
    for b in range(len(A)):
        check_rule(mon[b], steps[b], tol, T)
        Xf16, _, _ = cn(to_dev(A[b:b + 1]), to_dev(s[b:b + 1]), int(steps[b]), dash.DASH_FP16)
        assert rel_err(X[b], to_host(Xf16)[0])[0] <= 2e-3
        if LAM_MIN[b] >= 1e-2:  # binary16 storage error grows with the condition number
            Xo, _ = oracle.cn_inverse_root(A[b], 1.0, int(steps[b]))
            assert rel_err(X[b], Xo)[0] <= 5e-3
    assert np.all(np.diff(steps) >= 0) and steps[0] < steps[-1]
    well = np.array(LAM_MIN) >= 1e-2  # where binary16 storage keeps the monitor close to the residual
    assert np.all(residual(X[well], A[well]) <= 2.5 * tol)
