"""Pins of the CPU oracle against what the mathematics fixes (no GPU).

Each test checks the oracle against something other than itself: closed forms derived in exact
arithmetic (tests/golden/closed_forms.json), library routines on special cases (numpy's eigh,
float16 conversion, Chebyshev interpolation), brute force on 4x4 blocks, defining invariants and
limits of each iteration, and exact integer arithmetic.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import dash_inputs as di
import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b))


def spd(seed, n, lam_min, lam_max):
    A, Q, lam = di.known_spectrum_stack(seed, 1, n, lam_min, lam_max)
    return A[0], Q[0], lam[0]


# ----------------------------------------------------------------------------------------------
# elementary routines
# ----------------------------------------------------------------------------------------------

def test_matmul_matches_library_product():
    g = di.rng(11)
    X, Y = g.standard_normal((7, 7)), g.standard_normal((7, 7))
    assert rel(oracle.matmul(X, Y), X @ Y) < 1e-14
    # non-commuting operands: a swapped operand order would fail
    assert rel(oracle.matmul(X, Y), Y @ X) > 1e-3


def test_round_binary16_matches_numpy():
    g = di.rng(12)
    vals = list(g.standard_normal(2000) * np.exp(g.uniform(-20, 12, 2000)))
    ulp1 = 2.0 ** -10
    vals += [0.0, -0.0, 1.0, 1 + ulp1 / 2, 1 + 3 * ulp1 / 2, 2049.0, 2051.0, 65504.0, 65519.99, 65520.0, 7e4,
             2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 * (1 - 2.0 ** -11), 6.1e-5, -5.96e-8, 1e-9]
    x = np.array(vals)
    got = oracle.round_binary16(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    assert math.isnan(oracle.round_binary16(np.array([np.nan]))[0])


def _bf16(x):
    """Library bfloat16 rounding (torch, round to nearest even from binary32) of float32-exact values."""
    import torch

    x = np.asarray(x, dtype=np.float64)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x, equal_nan=True)
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bfloat16_matches_library():
    """bfloat16 rounding against torch's conversion on float32-exact values over the whole exponent
    range, ties to even, the overflow threshold and the subnormal range."""
    g = di.rng(13)
    vals = list((g.standard_normal(3000) * np.exp(g.uniform(-95, 88, 3000))).astype(np.float32))
    ulp1 = 2.0 ** -7
    big = 2.0 ** 127
    vals += [0.0, -0.0, 1.0, 1 + ulp1 / 2, 1 + 3 * ulp1 / 2, -(1 + ulp1 / 2), 257.0, 259.0,
             (2 - ulp1) * big, (2 - 2.0 ** -8 - 2.0 ** -23) * big, 2.0 ** -126, 2.0 ** -133,
             3 * 2.0 ** -134, 2.0 ** -135, 2.0 ** -126 * (1 - 2.0 ** -8)]
    x = np.array(vals, dtype=np.float64)
    assert np.array_equal(oracle.round_bfloat16(x), _bf16(x))
    assert oracle.round_bfloat16(np.array([1 + ulp1 / 2]))[0] == 1.0  # tie to the even neighbour
    assert oracle.round_bfloat16(np.array([1 + 3 * ulp1 / 2]))[0] == 1 + 2 * ulp1
    top = oracle.round_bfloat16(np.array([(2 - 2.0 ** -8) * big, (2 - 2.0 ** -8) * big * (1 - 2.0 ** -30)]))
    assert math.isinf(top[0]) and top[1] == (2 - ulp1) * big  # halfway to 2^128 overflows, below it does not
    assert math.isnan(oracle.round_bfloat16(np.array([np.nan]))[0])


# ----------------------------------------------------------------------------------------------
# c1: exact root by Jacobi eigendecomposition
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fx", GOLDEN["inverse_roots"], ids=lambda f: f["name"])
def test_power_evd_closed_forms(fx):
    A = np.array(fx["A"])
    assert rel(oracle.inverse_root_evd(A), fx["inv_fourth_root"]) < 1e-13
    assert rel(oracle.power_evd(A, 0.5), fx["sqrt"]) < 1e-13


def test_jacobi_diagonal_is_exact():
    d = np.array([3.0, -1.0, 7.5, 0.25, 2.0])
    w, Q, sweeps = oracle.jacobi_eigh(np.diag(d))
    assert sweeps == 0
    assert np.array_equal(w, d) and np.array_equal(Q, np.eye(5))


def test_jacobi_known_spectrum_and_invariants():
    A, Q, lam = spd(21, 40, 1e-3, 2.0)
    w, V, sweeps = oracle.jacobi_eigh(A)
    assert 0 < sweeps < 20
    assert np.max(np.abs(np.sort(w) - np.sort(lam))) < 1e-13 * np.linalg.norm(A)
    assert np.max(np.abs(V.T @ V - np.eye(40))) < 1e-13
    assert np.max(np.abs(A @ V - V * w[None, :])) < 1e-12


def test_jacobi_matches_numpy_eigh():
    g = di.rng(22)
    M = g.standard_normal((48, 48))
    A = M + M.T
    w, _, _ = oracle.jacobi_eigh(A)
    assert np.max(np.abs(np.sort(w) - np.linalg.eigvalsh(A))) < 1e-12 * np.abs(A).max() * 48


def _det_leibniz(M):
    n = len(M)
    tot = 0.0
    for perm in itertools.permutations(range(n)):
        sign = 1
        for i in range(n):
            for j in range(i + 1, n):
                if perm[i] > perm[j]:
                    sign = -sign
        prod = 1.0
        for i in range(n):
            prod *= M[i][perm[i]]
        tot += sign * prod
    return tot


def _brute_eigs_4x4(A):
    """Eigenvalues of a symmetric 4x4 by bisection on det(A - x I) (Leibniz determinant)."""
    radius = max(sum(abs(v) for v in row) for row in A)  # Gershgorin bound
    f = lambda x: _det_leibniz([[A[i][j] - (x if i == j else 0.0) for j in range(4)] for i in range(4)])
    grid = np.linspace(-radius - 1, radius + 1, 4001)
    vals = [f(x) for x in grid]
    roots = []
    for a, b, fa, fb in zip(grid[:-1], grid[1:], vals[:-1], vals[1:]):
        if fa == 0.0:
            roots.append(a)
        elif fa * fb < 0:
            for _ in range(200):
                m = 0.5 * (a + b)
                fm = f(m)
                if fa * fm <= 0:
                    b = m
                else:
                    a, fa = m, fm
            roots.append(0.5 * (a + b))
    return np.array(sorted(roots))


def _inverse_cofactor(A):
    n = len(A)
    det = _det_leibniz(A)
    inv = np.empty((n, n))
    for i in range(n):
        for j in range(n):
            minor = [[A[r][c] for c in range(n) if c != j] for r in range(n) if r != i]
            inv[j][i] = (-1) ** (i + j) * _det_leibniz(minor) / det
    return inv


def test_brute_force_4x4():
    g = di.rng(23)
    for _ in range(3):
        M = g.standard_normal((4, 4))
        A = M @ M.T + 0.5 * np.eye(4)  # SPD with well separated-enough eigenvalues
        w, _, _ = oracle.jacobi_eigh(A)
        assert np.max(np.abs(np.sort(w) - _brute_eigs_4x4(A.tolist()))) < 1e-10
        X = oracle.inverse_root_evd(A)
        X4 = X @ X @ X @ X
        assert rel(X4, _inverse_cofactor(A.tolist())) < 1e-12
        assert np.max(np.abs(X - X.T)) < 1e-14 and np.min(np.linalg.eigvalsh(X)) > 0


def test_power_evd_rejects_indefinite():
    with pytest.raises(ValueError):
        oracle.inverse_root_evd(np.diag([1.0, -0.5, 2.0]))


# ----------------------------------------------------------------------------------------------
# c2: Frobenius scale
# ----------------------------------------------------------------------------------------------

def test_frobenius_pins():
    assert oracle.frobenius(np.eye(64)) == 8.0
    A, _, lam = spd(24, 32, 1e-2, 3.0)
    s = oracle.frobenius(A)
    assert s == 0.25 * oracle.frobenius(-4.0 * A)
    assert s >= lam.max()
    assert abs(s - math.sqrt(np.sum(lam ** 2))) < 1e-13 * s  # ||A||_F^2 = sum of squared eigenvalues
    st = oracle.frobenius(np.stack([np.eye(16), 2 * np.eye(16)]))
    assert np.array_equal(st, [4.0, 8.0])


# ----------------------------------------------------------------------------------------------
# c3: Multi-Power-Iteration
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fx", GOLDEN["power_iteration"], ids=lambda f: "T%d_n%d" % (f["T"], len(f["lam"])))
def test_mpi_closed_form_fixtures(fx):
    A = np.diag(fx["lam"])
    s, mu = oracle.mpi(A, np.array(fx["V0"]), fx["T"])
    assert np.max(np.abs(mu - fx["mu"]) / np.abs(fx["mu"])) < 1e-14
    assert abs(s - fx["s"]) <= 1e-14 * fx["s"]


def test_mpi_closed_form_known_spectrum():
    A, Q, lam = spd(25, 48, 1e-3, 1.0)
    V0 = di.start_vectors(48, 8, seed=26).astype(np.float64)
    U = Q.T @ V0
    for T in (1, 3, 10):
        s, mu = oracle.mpi(A, V0, T)
        want = (lam[:, None] ** (2 * T - 1) * U ** 2).sum(0) / (lam[:, None] ** (2 * T - 2) * U ** 2).sum(0)
        assert np.max(np.abs(mu - want) / want) < 1e-12
        assert s == mu.max()


def test_mpi_bounds_monotone_and_identity():
    A, _, lam = spd(27, 64, 1e-4, 1.0)
    V0 = di.start_vectors(64, 32, seed=28)
    prev = 0.0
    for T in range(1, 12):
        s, mu = oracle.mpi(A, V0, T)
        assert np.all(mu <= lam.max() * (1 + 1e-14))
        assert s >= prev * (1 - 1e-14)  # Rayleigh quotients of the power iteration never decrease
        prev = s
    s, _ = oracle.mpi(3.25 * np.eye(32), di.start_vectors(32, 4, seed=29), 10)
    assert abs(s - 3.25) < 1e-15 * 3.25


def test_mpi_half_precision():
    # A = 2^m I: the binary16 operand is exactly I, every Rayleigh quotient is exactly 1, s = 2^m
    s, mu = oracle.mpi(np.eye(32) * 2.0 ** -7, di.start_vectors(32, 5, seed=30), 6, half=True)
    assert s == 2.0 ** -7 and np.all(mu == 2.0 ** -7)
    # close to the fp64 estimate on a well conditioned block (binary16 storage of A and V)
    A = di.tiny_stack()[0].astype(np.float64)
    V0 = di.start_vectors(64, 32)
    s64, _ = oracle.mpi(A, V0, 10)
    s16, _ = oracle.mpi(A, V0, 10, half=True)
    assert abs(s16 - s64) / s64 < 2e-3
    # zero block: no positive diagonal, scale 0
    assert oracle.mpi(np.zeros((8, 8)), np.ones((8, 2)), 3, half=True)[0] == 0.0


def _mpi_half_diagonal(a, V0, T, prescale="ceil", round_w=False):
    """The binary16 power iteration on diag(a), written as its scalar recurrence with numpy's float16
    (round to nearest even): e = ceil(log2 max a), a_h = fp16(a 2^-e), v = fp16(v0 / |v0|), and per
    step w = a_h v (exact), mu = 2^e (v.w)/(v.v), v <- fp16(w / |w|).  The planted variants prescale
    by 2^-floor(log2 max a), or round w before it is normalised."""
    f16 = lambda x: np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    m = float(np.max(a))
    e = math.ceil(math.log2(m)) if prescale == "ceil" else math.floor(math.log2(m))
    ah = f16(a * 2.0 ** -e)
    V = f16(V0 / np.linalg.norm(V0, axis=0))
    for t in range(1, T + 1):
        W = ah[:, None] * V
        mu = 2.0 ** e * np.sum(V * W, axis=0) / np.sum(V * V, axis=0)
        if t < T:
            if round_w:
                Wr = f16(W)
                V = Wr / np.linalg.norm(Wr, axis=0)
            else:
                V = f16(W / np.linalg.norm(W, axis=0))
    return mu.max(), mu


def test_mpi_half_diagonal_matches_scalar_recurrence():
    """Pins where the binary16 power iteration rounds: on a diagonal block every step is the scalar
    recurrence above.  The block's largest entry 3 has ceil(log2 3) = 2 != floor(log2 3) = 1, and half
    of its entries lie in [2^-13, 2^-12), which the ceil prescale takes into binary16's subnormal range
    and the floor prescale does not, so a floor prescale changes the result; so does rounding w before
    its normalisation."""
    g = di.rng(61)
    n, k = 64, 4
    a = np.concatenate([[3.0], g.uniform(0.1, 2.9, n // 4 - 1), g.uniform(2.0 ** -13, 2.0 ** -12, 3 * n // 4)])
    a = a[g.permutation(n)]
    V0 = di.start_vectors(n, k, seed=62).astype(np.float64)
    for T in (1, 2, 3, 10):
        s, mu = oracle.mpi(np.diag(a), V0, T, half=True)
        s_ref, mu_ref = _mpi_half_diagonal(a, V0, T)
        assert np.allclose(mu, mu_ref, rtol=1e-13, atol=0), T
        assert abs(s - s_ref) <= 1e-13 * s_ref
    # the planted variants disagree with the oracle by far more than the pin's tolerance
    s, mu = oracle.mpi(np.diag(a), V0, 1, half=True)
    _, mu_floor = _mpi_half_diagonal(a, V0, 1, prescale="floor")
    assert np.max(np.abs(mu_floor - mu) / mu) > 1e-11
    for T in (2, 3):
        s, mu = oracle.mpi(np.diag(a), V0, T, half=True)
        _, mu_w = _mpi_half_diagonal(a, V0, T, round_w=True)
        assert np.max(np.abs(mu_w - mu) / mu) > 1e-9, T


# ----------------------------------------------------------------------------------------------
# per-block interval bottom, residual probe and routing
# ----------------------------------------------------------------------------------------------

def test_mpi_shifted_closed_form_on_diagonal():
    """On diag(lam) the shifted iteration's Rayleigh quotients have the closed form of the power
    iteration on diag(c), c = sigma - lam: mu_j = sum c^(2T-1) u_j^2 / sum c^(2T-2) u_j^2, evaluated
    here in exact rational arithmetic."""
    from fractions import Fraction

    lam = [Fraction(1, 8), Fraction(1, 2), Fraction(3, 4), Fraction(1, 1), Fraction(5, 4), Fraction(3, 2)]
    sigma = Fraction(2)
    U = [[1, 2, -1], [2, 0, 1], [-1, 1, 3], [3, -2, 1], [1, 1, 1], [2, -1, 2]]
    A = np.diag([float(x) for x in lam])
    V0 = np.array(U, dtype=np.float64)
    for T in (1, 3, 7):
        lam_hat, mu = oracle.mpi_shifted(A, float(sigma), V0, T)
        exact = []
        for j in range(3):
            c = [sigma - x for x in lam]
            num = sum(ci ** (2 * T - 1) * U[i][j] ** 2 for i, ci in enumerate(c))
            den = sum(ci ** (2 * T - 2) * U[i][j] ** 2 for i, ci in enumerate(c))
            exact.append(num / den)
        assert np.allclose(mu, [float(x) for x in exact], rtol=1e-14, atol=0)
        assert abs(lam_hat - float(sigma - max(exact))) < 1e-14


def test_mpi_shifted_bounds_and_limit():
    """The estimate lies above lambda_min, falls with every step, and reaches it when the bottom
    eigenvalue is well separated."""
    A, _, lam = spd(63, 48, 0.02, 1.0)
    V0 = di.start_vectors(48, 32, seed=64)
    prev = np.inf
    for T in (1, 2, 4, 8, 16):
        est, _ = oracle.mpi_shifted(A, 1.25, V0, T)
        assert est >= lam.min() * (1 - 1e-12)
        assert est <= prev * (1 + 1e-14)
        prev = est
    g = di.rng(65)
    lam2 = np.concatenate([[0.01], g.uniform(0.5, 1.0, 47)])
    Q = di.haar_orthogonal(g, 48)
    A2 = (Q * lam2[None, :]) @ Q.T
    est, _ = oracle.mpi_shifted(0.5 * (A2 + A2.T), 1.25, V0, 200)
    assert abs(est - 0.01) < 1e-10


def test_residual_probe_closed_form_and_expectation():
    g = di.rng(66)
    n, k = 40, 6
    a = g.uniform(0.1, 1.0, n)
    x = a ** -0.25 * (1.0 + g.uniform(-0.01, 0.01, n))
    V0 = di.start_vectors(n, k, seed=67).astype(np.float64)
    # diagonal blocks: E = diag(x^4 a - 1), so ||E v||^2 = sum_i e_i^2 v_i^2 for each unit probe v
    r = oracle.residual_probe(np.diag(a), np.diag(x), V0)
    e = x ** 4 * a - 1.0
    v = V0 / np.sqrt(np.sum(V0 * V0, axis=0))
    assert abs(r - math.sqrt(np.mean(np.sum((e[:, None] * v) ** 2, axis=0)))) < 1e-14
    # the exact root (closed form) has no residual
    A, Q, lam = spd(68, 32, 1e-3, 1.0)
    X = (Q * lam[None, :] ** -0.25) @ Q.T
    assert oracle.residual_probe(A, X, di.start_vectors(32, 8, seed=69)) < 1e-11
    # many probes: the mean of ||E v||^2 over the sphere is ||E||_F^2 / n
    Xp = X + 1e-3 * (g.standard_normal((32, 32)))
    E = np.linalg.matrix_power(Xp, 4) @ A - np.eye(32)
    r_exact = np.linalg.norm(E) / math.sqrt(32)
    r_many = oracle.residual_probe(A, Xp, g.standard_normal((32, 4000)))
    assert abs(r_many - r_exact) < 0.05 * r_exact


def test_cheb_interval_lo_and_per_block_lower_end():
    s = np.array([2.0, 4.0, 8.0])
    lo = oracle.cheb_interval_lo(s, 0.1)
    assert np.array_equal(lo, [0.05, 0.025, 0.0125])
    lo = oracle.cheb_interval_lo(s, 0.1, lam=[1.0, 0.1, np.nan], theta=0.5)
    assert np.allclose(lo, [0.25, 0.025, 0.0125], rtol=0, atol=0)  # a NaN estimate leaves the floor
    # a per-block lower end gives each block the solve it would get alone
    A, _, _ = spd(70, 24, 0.05, 1.0)
    B2, _, _ = spd(71, 24, 0.2, 1.0)
    X = oracle.cheb_inverse_root(np.stack([A, B2]), [1.0, 1.0], 10, [0.04, 0.15], 1.25)
    assert np.array_equal(X[0], oracle.cheb_inverse_root(A, 1.0, 10, 0.04, 1.25))
    assert np.array_equal(X[1], oracle.cheb_inverse_root(B2, 1.0, 10, 0.15, 1.25))


def test_routed_inverse_root_routes_and_meets_the_gate():
    """A well-conditioned block stays with Chebyshev on its estimated interval; a kappa = 1e4 block,
    whose floor-based interval leaves degree 16 far from the gate, goes to coupled Newton; both meet
    the fp32 residual gate against the closed-form root."""
    n = 48
    A0, Q0, l0 = spd(72, n, 0.25, 1.0)
    A1, Q1, l1 = spd(73, n, 1e-4, 1.0)
    A = np.stack([A0, A1])
    s = np.array([l0.max(), l1.max()]) / 1.02
    V0 = di.start_vectors(n, 16, seed=74).astype(np.float64)
    X, route, lam, r = oracle.routed_inverse_root(A, s, 16, 0.9e-4, 1.25, V0, 10, 1e-3, 30)
    assert list(route) == [0, 1]
    assert np.all(lam >= np.array([l0.min(), l1.min()]) * (1 - 1e-12))
    assert r[0] < 1e-5 and r[1] > 1e-3
    for b, (Q, l) in enumerate(((Q0, l0), (Q1, l1))):
        Xe = (Q * l[None, :] ** -0.25) @ Q.T
        E = np.linalg.matrix_power(X[b], 4) @ A[b] - np.eye(n)
        assert np.linalg.norm(E) / math.sqrt(n) < 1e-3
        assert rel(X[b], Xe) < 1e-3


# ----------------------------------------------------------------------------------------------
# c4 / c5: Newton-Denman-Beavers
# ----------------------------------------------------------------------------------------------

def test_ndb_identity_is_fixed_point():
    Y, Z, mon = oracle.ndb(np.eye(16), 5)
    assert np.array_equal(Y, np.eye(16)) and np.array_equal(Z, np.eye(16)) and np.all(mon == 0)


def test_ndb_limits_and_coupling_invariant():
    M, _, _ = spd(31, 32, 0.02, 1.0)
    R = oracle.power_evd(M, 0.5)
    Ri = oracle.power_evd(M, -0.5)
    for T in (1, 2, 4):
        Y, Z, _ = oracle.ndb(M, T)
        # coupled Denman-Beavers iterates satisfy Y_k = M Z_k and commute
        assert rel(Y, M @ Z) < 1e-13
        assert rel(Y @ Z, Z @ Y) < 1e-13
    Y, Z, mon = oracle.ndb(M, 25)
    assert rel(Y, R) < 1e-12 and rel(Z, Ri) < 1e-12
    assert rel(Y @ Y, M) < 1e-12 and rel(Y @ Z, np.eye(32)) < 1e-12
    # quadratic convergence of the monitor ||P - I||/sqrt(B) once it is small
    k = int(np.argmax(mon < 1e-2))
    assert mon[k + 1] < 10 * mon[k] ** 2


def test_ndb_stable_at_kappa_1e4():
    """The operand order (P = Z Y, Y' = Y S, Z' = S Z) stays converged long after convergence."""
    M, _, _ = spd(32, 64, 1e-4, 1.0)
    R = oracle.power_evd(M, 0.5)
    Y, Z, mon = oracle.ndb(M, 80)
    assert rel(Y, R) < 1e-10
    assert mon[-1] < 1e-12


def _ndb_numpy_swapped(M, T):
    """A planted mistake (for the test above to catch): Y' = S Y instead of Y S."""
    Y, Z = M.copy(), np.eye(len(M))
    for _ in range(T):
        S = 1.5 * np.eye(len(M)) - 0.5 * (Z @ Y)
        Y, Z = S @ Y, S @ Z
    return Y


def test_ndb_stability_pin_catches_swapped_order():
    M, _, _ = spd(32, 64, 1e-4, 1.0)
    R = oracle.power_evd(M, 0.5)
    with np.errstate(all="ignore"):
        bad = _ndb_numpy_swapped(M, 80)
    assert not np.all(np.isfinite(bad)) or rel(bad, R) > 1e-6


@pytest.mark.parametrize("fx", GOLDEN["inverse_roots"], ids=lambda f: f["name"])
def test_ndb_inverse_root_closed_forms(fx):
    A = np.array(fx["A"])
    X, R, mon = oracle.ndb_inverse_root(A, fx["lambda_max"], 30, 30, want_sqrt=True)
    assert rel(X, fx["inv_fourth_root"]) < 1e-12
    assert rel(R, fx["sqrt"]) < 1e-12
    assert mon.shape == (60,)


def test_ndb_inverse_root_tiny_stack_and_scale_equivariance():
    A = di.tiny_stack().astype(np.float64)
    s, _ = oracle.mpi(A, di.start_vectors(64, 32), 10)
    X, _, _ = oracle.ndb_inverse_root(A, s, 20, 20)
    assert rel(X, oracle.inverse_root_evd(A)) < 1e-10
    X16, _, _ = oracle.ndb_inverse_root(16 * A, 16 * s, 20, 20)
    assert rel(2 * X16, X) < 1e-15


# ----------------------------------------------------------------------------------------------
# c6: Coupled Newton, p = 4
# ----------------------------------------------------------------------------------------------

def test_cn_identity():
    X, mon = oracle.cn_inverse_root(16.0 * np.eye(8), 16.0, 4)
    assert np.array_equal(X, 0.5 * np.eye(8)) and np.all(mon == 0)
    Xh, _ = oracle.cn_inverse_root(16.0 * np.eye(8), 16.0, 4, half_storage=True)
    assert np.array_equal(Xh, 0.5 * np.eye(8))


def test_cn_monitor_is_residual_and_limit():
    A, _, _ = spd(41, 32, 1e-3, 1.0)
    exact = oracle.inverse_root_evd(A)
    for T in (1, 2, 3, 5):
        X, mon = oracle.cn_inverse_root(A, 1.0, T)
        # in exact arithmetic M_k = X_k^4 A_s, so the monitor of step T (one more step) is the residual
        X2, mon2 = oracle.cn_inverse_root(A, 1.0, T + 1)
        r = np.linalg.norm(X @ X @ X @ X @ A - np.eye(32)) / math.sqrt(32)
        assert abs(mon2[T] - r) < 1e-10 * max(r, 1e-3)
    X, mon = oracle.cn_inverse_root(A, 1.0, 40)
    assert rel(X, exact) < 1e-10


@pytest.mark.parametrize("fx", GOLDEN["inverse_roots"], ids=lambda f: f["name"])
def test_cn_closed_forms(fx):
    A = np.array(fx["A"])
    X, _ = oracle.cn_inverse_root(A, fx["lambda_max"], 40)
    assert rel(X, fx["inv_fourth_root"]) < 1e-12


def test_cn_half_storage_residual():
    A = di.tiny_stack()[:2].astype(np.float64)
    s, _ = oracle.mpi(A, di.start_vectors(64, 32), 10)
    X, _ = oracle.cn_inverse_root(A, s, 8, half_storage=True)
    for b in range(2):
        r = np.linalg.norm(np.linalg.matrix_power(X[b], 4) @ A[b] - np.eye(64)) / 8.0
        assert r < 5e-3


# ----------------------------------------------------------------------------------------------
# c7: Chebyshev / Clenshaw
# ----------------------------------------------------------------------------------------------

# ---- NDB with binary16 iterates and fp32 correction (reading: stored iterates rounded to binary16,
# exact products; correction X <- sym(X (5I - X^4 A_s)/4))

_ROUND = {"binary16": lambda x: float(np.float16(x)), "bfloat16": lambda x: float(_bf16([x])[0])}


def _scalar_ndb_half(m, T, keep_last, h):
    z = h(1.5 - 0.5 * m)
    y = h(m * z)
    for k in range(1, T):
        sc = h(1.5 - 0.5 * (z * y))
        y = h(y * sc)
        z = sc * z if (keep_last and k == T - 1) else h(sc * z)
    return y, z


@pytest.mark.parametrize("storage", ["binary16", "bfloat16"])
def test_ndb_half_diagonal_matches_scalar_recurrence(storage):
    """On diagonal blocks every product is an exact product of 2-byte numbers, so the scalar
    recurrence with the same roundings (numpy float16, or torch's bfloat16 conversion, both round to
    nearest even; every rounded value is exact in float32, so neither rounds twice) gives the
    oracle's result exactly; so does the scalar correction step.  s is a power of two and the
    eigenvalues are float32 numbers, so A/s is exact before its first rounding."""
    h = _ROUND[storage]
    lam = np.exp(np.linspace(np.log(0.05), 0.0, 16)).astype(np.float32).astype(np.float64)
    s = 2.0
    for T1, T2, refine in ((6, 6, 0), (5, 4, 2), (1, 1, 1)):
        X = oracle.ndb_half_inverse_root(np.diag(lam), s, T1, T2, refine, storage=storage)
        assert np.count_nonzero(X - np.diag(np.diag(X))) == 0
        xs, ms = [], []
        for l in lam:
            m = l / s
            y, _ = _scalar_ndb_half(h(m), T1, False, h)
            _, x = _scalar_ndb_half(y, T2, True, h)
            xs.append(x)
            ms.append(m)

        def tvals(xv):  # T = (5 - x^4 m)/4 per entry, and the block's residual 4 ||T - 1||_F / sqrt(n)
            t = [(5.0 - ((xi * xi) * (xi * xi)) * mi) / 4.0 for xi, mi in zip(xv, ms)]
            return t, 4.0 * math.sqrt(sum((ti - 1.0) ** 2 for ti in t) / len(t))

        t, r_cur = tvals(xs)
        for _ in range(refine):  # guarded: a step is taken only if the residual goes down
            xc = [xi * ti for xi, ti in zip(xs, t)]
            tc, r_c = tvals(xc)
            if not r_c < r_cur:
                break
            xs, t, r_cur = xc, tc, r_c
        for i in range(len(lam)):
            assert X[i, i] == s ** -0.25 * xs[i]


@pytest.mark.parametrize("storage", ["binary16", "bfloat16"])
def test_cn_storage_diagonal_matches_scalar_recurrence(storage):
    """Coupled Newton with 2-byte storage on diagonal blocks: each diagonal entry follows the scalar
    recurrence S = h((5 - m)/4), x = h(x S) (the last x unrounded), m = h(m h(h(S S)^2)), all
    products exact in float64 (and in float32 before rounding)."""
    h = _ROUND[storage]
    lam = np.exp(np.linspace(np.log(0.02), 0.0, 12)).astype(np.float32).astype(np.float64)
    s = 2.0
    T = 6
    X, mon = oracle.cn_inverse_root(np.diag(lam), s, T, storage=storage)
    assert np.count_nonzero(X - np.diag(np.diag(X))) == 0
    for i, l in enumerate(lam):
        m, x = h(l / s), 1.0
        for k in range(T):
            sk = h((5.0 - m) / 4.0)
            x = x * sk if k == T - 1 else h(x * sk)
            s2 = h(sk * sk)
            m = h(m * h(s2 * s2))
        assert X[i, i] == s ** -0.25 * x
    # the exact iteration differs: the storage rounding is what the model adds
    X_exact, _ = oracle.cn_inverse_root(np.diag(lam), s, T)
    assert not np.array_equal(X, X_exact)


def test_ndb_half_guard_stops_a_diverging_correction():
    """At kappa ~25-35 the plain Newton correction diverges (the residual grows step by step, as the
    unguarded steps computed here show); the guarded correction then never ends worse than its
    start."""
    A = di.tiny_stack().astype(np.float64)
    s = np.linalg.eigvalsh(A)[:, -1] * 1.02
    X0 = oracle.ndb_half_inverse_root(A, s, 6, 6, 0)
    Xg = oracle.ndb_half_inverse_root(A, s, 6, 6, 4)
    diverged = 0
    for b in range(A.shape[0]):
        As = A[b] / s[b]
        x = X0[b] * s[b] ** 0.25
        rs = []
        for _ in range(3):
            rs.append(np.linalg.norm(np.linalg.matrix_power(x, 4) @ As - np.eye(64)))
            x = x @ ((5 * np.eye(64) - np.linalg.matrix_power(x, 4) @ As) / 4)
            x = 0.5 * (x + x.T)
        r_g = np.linalg.norm(np.linalg.matrix_power(Xg[b], 4) @ A[b] - np.eye(64))
        assert r_g <= rs[0] * (1 + 1e-12)
        diverged += rs[2] > rs[0]
    assert diverged >= 1


def test_ndb_half_residual_and_correction():
    """Binary16 NDB meets the binary16 gate at kappa ~5, and each correction step lowers the
    residual and the distance to the exact root."""
    g = di.rng(77)
    G = g.standard_normal((96, 96)) * 1e-3
    A = G @ G.T / 96 + 1e-6 * np.eye(96)
    s = np.linalg.eigvalsh(A)[-1] * 1.02
    exact = oracle.inverse_root_evd(A)
    prev_r, prev_e = None, None
    for refine in range(4):
        X = oracle.ndb_half_inverse_root(A, s, 6, 6, refine)
        X2 = X @ X
        r = np.linalg.norm(X2 @ X2 @ A - np.eye(96)) / np.sqrt(96)
        e = np.linalg.norm(X - exact) / np.linalg.norm(exact)
        if refine == 0:
            assert r < 5e-3
        else:
            assert r < prev_r and e < prev_e
            assert np.array_equal(X, X.T)
        prev_r, prev_e = r, e


# ---- adaptive stopping rule ([PT] Significância e Alegações, "Direções Futuras"; reading: a call
# stops before step k >= 1 once its monitor is <= tol)

def _scalar_ndb_monitors(m, T):
    """Monitors of one NDB call on diag(m), from the scalar recurrence per eigenvalue (plain floats)."""
    y, z, mons = list(m), [1.0] * len(m), []
    for _ in range(T):
        p = [zi * yi for zi, yi in zip(z, y)]
        mons.append(math.sqrt(sum((pi - 1.0) ** 2 for pi in p) / len(p)))
        sc = [(3.0 - pi) / 2.0 for pi in p]
        y = [yi * si for yi, si in zip(y, sc)]
        z = [si * zi for si, zi in zip(sc, z)]
    return mons, y


def _scalar_cn_monitors(m, T):
    x, mm, mons = [1.0] * len(m), list(m), []
    for _ in range(T):
        mons.append(math.sqrt(sum((mi - 1.0) ** 2 for mi in mm) / len(mm)))
        sc = [(5.0 - mi) / 4.0 for mi in mm]
        x = [xi * si for xi, si in zip(x, sc)]
        mm = [mi * si ** 4 for mi, si in zip(mm, sc)]
    return mons


def _first_below(mons, tol, T):
    return next((k for k in range(1, T) if mons[k] <= tol), T)


def test_adaptive_step_counts_closed_form():
    """Diagonal blocks: the scalar recurrences give every monitor, hence the step at which each call
    stops; tol sits midway (in log scale) between two consecutive monitors of the deciding step."""
    lam = np.exp(np.linspace(np.log(3e-3), 0.0, 48))
    A = np.diag(lam)
    T = 25
    mons1, y = _scalar_ndb_monitors(list(lam), T)
    k1 = _first_below(mons1, 1e-3, T)
    tol = math.sqrt(mons1[k1] * mons1[k1 - 1])        # between the last monitor above and the first below
    X, mon, steps = oracle.ndb_inverse_root_adaptive(A, 1.0, T, T, tol)
    assert steps[0] == _first_below(mons1, tol, T)
    y1, _ = _scalar_ndb_monitors(list(lam), steps[0])[1], None
    mons2, _ = _scalar_ndb_monitors(y1, T)
    assert steps[1] == _first_below(mons2, tol, T)
    np.testing.assert_allclose(mon[: steps[0] + 1], mons1[: steps[0] + 1], rtol=1e-9, atol=1e-15)
    assert np.all(mon[steps[0] + 1:T] == 0.0)
    monc = _scalar_cn_monitors(list(lam), T)
    kc = _first_below(monc, 1e-3, T)
    tolc = math.sqrt(monc[kc] * monc[kc - 1])
    Xc, monc_o, stc = oracle.cn_inverse_root_adaptive(A, 1.0, T, tolc)
    assert stc == _first_below(monc, tolc, T)
    np.testing.assert_allclose(monc_o[: stc + 1], monc[: stc + 1], rtol=1e-9, atol=1e-15)


def test_adaptive_equals_fixed_run_of_its_length():
    """Stopping after k steps leaves exactly the k-step result (bitwise), and the step count is the
    first k >= 1 whose fixed-run monitor is <= tol; tol < 0 never stops."""
    A = di.tiny_stack()
    s = np.array([np.linalg.norm(a) for a in A])
    tol = 1e-6
    X, mon, steps = oracle.ndb_inverse_root_adaptive(A, s, 20, 20, tol)
    for b in range(A.shape[0]):
        Xf, _, monf = oracle.ndb_inverse_root(A[b], s[b], int(steps[b, 0]), int(steps[b, 1]))
        assert np.array_equal(X[b], Xf)
        _, _, mon_full1 = oracle.ndb_inverse_root(A[b], s[b], 20, 1)
        assert steps[b, 0] == _first_below(list(mon_full1[:20]), tol, 20)
    Xc, monc, stc = oracle.cn_inverse_root_adaptive(A, s, 20, tol)
    for b in range(A.shape[0]):
        Xf, monf = oracle.cn_inverse_root(A[b], s[b], int(stc[b]))
        assert np.array_equal(Xc[b], Xf)
        _, mon_full = oracle.cn_inverse_root(A[b], s[b], 20)
        assert stc[b] == _first_below(list(mon_full), tol, 20)
    Xn, _, stn = oracle.ndb_inverse_root_adaptive(A, s, 6, 5, -1.0)
    assert np.all(stn == [6, 5])
    assert np.array_equal(Xn, oracle.ndb_inverse_root(A, s, 6, 5)[0])


@pytest.mark.parametrize("fx", GOLDEN["chebyshev"], ids=lambda f: "%g_%g" % (f["lo"], f["hi"]))
def test_cheb_coeffs_x2_closed_form(fx):
    c = oracle.cheb_coeffs(2, fx["lo"], fx["hi"], 2.0)
    assert np.max(np.abs(c - fx["coeffs"])) < 1e-13 * max(1.0, np.abs(fx["coeffs"]).max())
    c5 = oracle.cheb_coeffs(5, fx["lo"], fx["hi"], 2.0)
    assert np.max(np.abs(c5[:3] - fx["coeffs"])) < 1e-12 * max(1.0, np.abs(fx["coeffs"]).max())
    assert np.max(np.abs(c5[3:])) < 1e-12 * max(1.0, np.abs(fx["coeffs"]).max())


def test_cheb_coeffs_match_numpy_interpolant():
    lo, hi, d = 1e-3, 1.25, 24
    c = oracle.cheb_coeffs(d, lo, hi, -0.25)
    ref = np.polynomial.chebyshev.chebinterpolate(lambda t: (((hi - lo) * t + hi + lo) / 2) ** -0.25, d)
    assert np.max(np.abs(c - ref)) < 1e-12 * np.abs(ref).max()
    # interpolation property at the nodes
    j = np.arange(d + 1)
    t = np.cos(np.pi * (j + 0.5) / (d + 1))
    x = ((hi - lo) * t + hi + lo) / 2
    assert np.max(np.abs(np.polynomial.chebyshev.chebval(t, c) / x ** -0.25 - 1)) < 1e-12


def test_clenshaw_scalar_and_x2():
    lo, hi = 0.1, 1.3
    c = oracle.cheb_coeffs(9, lo, hi, -0.25)
    for a in (0.1, 0.37, 1.0, 1.3):
        t = (2 * a - lo - hi) / (hi - lo)
        want = sum(ck * math.cos(k * math.acos(t)) for k, ck in enumerate(c))
        assert abs(oracle.clenshaw(np.array([[a]]), c, lo, hi)[0, 0] - want) < 1e-14
    A, _, _ = spd(51, 24, 0.05, 1.0)
    c2 = oracle.cheb_coeffs(3, 0.0, 1.0, 2.0)
    assert rel(oracle.clenshaw(A, c2, 0.0, 1.0), A @ A) < 1e-13


def test_clenshaw_known_spectrum_and_cheb_root_error():
    A, Q, lam = spd(52, 32, 0.05, 1.0)
    lo, hi, d = 0.04, 1.1, 12
    c = oracle.cheb_coeffs(d, lo, hi, -0.25)
    P = oracle.clenshaw(A, c, lo, hi)
    p = np.polynomial.chebyshev.chebval((2 * lam - lo - hi) / (hi - lo), c)
    assert rel(P, (Q * p[None, :]) @ Q.T) < 1e-13
    # spectral-norm error of the matrix function equals the scalar error on the spectrum
    X = oracle.cheb_inverse_root(2.0 * A, 2.0, d, lo, hi)
    E = X - oracle.inverse_root_evd(2.0 * A)
    scalar = np.max(np.abs(p - lam ** -0.25)) * 2.0 ** -0.25
    assert abs(np.linalg.norm(E, 2) - scalar) < 1e-12


# ----------------------------------------------------------------------------------------------
# c8, c9, stacking
# ----------------------------------------------------------------------------------------------

def test_update_stats_exact_integers():
    g = di.rng(61)
    n = 12
    G = g.integers(-3, 4, (n, n)).astype(np.int64)
    L0 = g.integers(-5, 6, (n, n)).astype(np.int64)
    L0 = L0 + L0.T
    R0 = g.integers(-5, 6, (n, n)).astype(np.int64)
    R0 = R0 + R0.T
    L, R = oracle.update_stats(G, 0.5, L0, R0)
    assert np.array_equal(2 * L, L0 + G @ G.T)   # beta = 1/2 keeps every value exact
    assert np.array_equal(2 * R, R0 + G.T @ G)
    assert np.array_equal(L, L.T) and np.array_equal(R, R.T)
    # R(G) = L(G^T)
    L_t, _ = oracle.update_stats(G.T, 0.5, R0, L0)
    assert np.array_equal(L_t, R)


def test_apply_identity_and_integers():
    g = di.rng(62)
    G = g.standard_normal((3, 16, 16))
    I = np.broadcast_to(np.eye(16), G.shape)
    assert np.array_equal(oracle.apply(I, G, I), G)
    XL = g.integers(-3, 4, (3, 16, 16)).astype(np.int64)
    XR = g.integers(-3, 4, (3, 16, 16)).astype(np.int64)
    Gi = g.integers(-3, 4, (3, 16, 16)).astype(np.int64)
    assert np.array_equal(oracle.apply(XL, Gi, XR), XL @ Gi @ XR)
    assert not np.array_equal(oracle.apply(XL, Gi, XR), XR @ Gi @ XL)


def test_stack_order_and_round_trip():
    B = 4
    shapes = [(8, 12), (4, 4), (12, 8)]
    g = di.rng(63)
    W = [g.standard_normal(s) for s in shapes]
    S = oracle.stack(W, B)
    assert S.shape == (6 + 1 + 6, B, B)
    # tile (tr, tc) of weight w sits at offset(w) + tr * (cols / B) + tc
    assert np.array_equal(S[0], W[0][0:4, 0:4])
    assert np.array_equal(S[2], W[0][0:4, 8:12])
    assert np.array_equal(S[3], W[0][4:8, 0:4])
    assert np.array_equal(S[6], W[1])
    assert np.array_equal(S[7 + 2 * 2 + 1], W[2][8:12, 4:8])
    back = oracle.unstack(S, shapes, B)
    assert all(np.array_equal(a, b) for a, b in zip(back, W))
    with pytest.raises(ValueError):
        oracle.stack([np.zeros((0, 8))], B)


def test_stack_edge_tiles_are_zero_padded():
    # sides that are not multiples of B: ceil(rows/B) x ceil(cols/B) tiles, zero outside the weight
    B = 4
    shapes = [(6, 9), (3, 2), (4, 5)]
    g = di.rng(64)
    W = [g.standard_normal(s) for s in shapes]
    S = oracle.stack(W, B)
    assert S.shape == (2 * 3 + 1 + 1 * 2, B, B) and di.num_tiles(shapes, B) == 9
    assert np.array_equal(S[0], W[0][0:4, 0:4])
    assert np.array_equal(S[2][:4, :1], W[0][0:4, 8:9]) and not S[2][:, 1:].any()
    assert np.array_equal(S[5][:2, :1], W[0][4:6, 8:9]) and not S[5][2:].any() and not S[5][:, 1:].any()
    assert np.array_equal(S[6][:3, :2], W[1]) and not S[6][3:].any() and not S[6][:, 2:].any()
    assert np.array_equal(S[8][:, :1], W[2][:, 4:5]) and not S[8][:, 1:].any()
    # a padded tile's Gram products keep the padding zero, the valid part is the weight's own
    L, R = oracle.update_stats(S, 0.0, np.zeros_like(S), np.zeros_like(S))
    assert np.allclose(L[6][:3, :3], W[1] @ W[1].T) and not L[6][3:].any() and not L[6][:, 3:].any()
    assert np.allclose(R[6][:2, :2], W[1].T @ W[1]) and not R[6][2:].any() and not R[6][:, 2:].any()
    back = oracle.unstack(S, shapes, B)
    assert all(np.array_equal(a, b) for a, b in zip(back, W))


def test_llama_shapes_give_1536_tiles():
    assert di.num_tiles(di.llama_weight_shapes(), 1024) == 1536


# ----------------------------------------------------------------------------------------------
# 1-D parameters
# ----------------------------------------------------------------------------------------------

def test_vec_pieces_round_trip_and_padding():
    g = di.rng(80)
    vs = [g.standard_normal(n) for n in (5, 64, 130, 1)]
    P = oracle.stack_vec(vs, 64)
    assert P.shape == (1 + 1 + 3 + 1, 64)
    assert np.array_equal(P[0, :5], vs[0]) and np.all(P[0, 5:] == 0)
    assert np.array_equal(P[2:5].reshape(-1)[:130], vs[2]) and np.all(P[4, 2:] == 0)
    back = oracle.unstack_vec(P, [5, 64, 130, 1], 64)
    assert all(np.array_equal(a, b) for a, b in zip(back, vs))


def test_vec_stats_and_apply_exact_on_integers():
    """Small integers and beta = 1/2 keep every value exact: the rank-one update equals numpy's outer
    product, the apply numpy's matrix-vector product, and L stays exactly symmetric."""
    g = di.rng(81)
    gv = g.integers(-8, 9, (3, 16)).astype(np.float64)
    L0 = g.integers(-8, 9, (3, 16, 16)).astype(np.float64)
    L0 = L0 + np.swapaxes(L0, 1, 2)
    L = oracle.update_stats_vec(gv, 0.5, L0)
    for p in range(3):
        assert np.array_equal(L[p], 0.5 * L0[p] + 0.5 * np.outer(gv[p], gv[p]))
        assert np.array_equal(L[p], L[p].T)
    X = g.integers(-8, 9, (3, 16, 16)).astype(np.float64)
    u = oracle.apply_vec(X, gv)
    assert np.array_equal(u, np.einsum("pij,pj->pi", X, gv))
    assert np.array_equal(oracle.apply_vec(np.stack([np.eye(16)] * 3), gv), gv)


def test_ndb_inverse_sqrt_closed_form():
    """One NDB call's Z, unscaled by s^{-1/2}, is A^{-1/2} = Q diag(lam^{-1/2}) Q^T (exact rational-free
    closed form); a power-of-two scale of A and s scales X by the exact power of two."""
    A, Q, lam = spd(82, 24, 0.05, 1.0)
    X = oracle.ndb_inverse_sqrt(A, lam.max(), 20)
    assert rel(X, (Q * lam[None, :] ** -0.5) @ Q.T) < 1e-12
    X16 = oracle.ndb_inverse_sqrt(16 * A, 16 * lam.max(), 20)
    assert np.array_equal(4 * X16, X)
