"""GPU parity of the eigendecomposition solver (batched two-sided block Jacobi,
dash_inverse_root_evd) against the CPU oracle's cyclic-Jacobi eigendecomposition: the exact root
A^{-1/4} and the eigenvalues.

Gates as for the iterations: fp32 iterate parity ||X_gpu - X_oracle||_F / ||X_oracle||_F <= 1e-4
where the condition number allows it (the EVD is the exact root, so the oracle's exact root is the
target), the residual ||X^4 A - I||_F / sqrt(B) <= 1e-3 evaluated in fp64 on the host, and every
block's eigenvalues within 2e-5 ||A||_2 of the oracle's.  With binary16 operands in the first pass
(dash_inverse_root_evd_prec, DASH_FP16, always refined) the gate is the binary16 one, residual
<= 5e-3, and the iterate is compared with the oracle's exact root to 1e-3; on the well-conditioned
stacks the binary16 solve is held to the fp32 gates as well (its products' errors scale with the
rotations' distance from the identity).
"""
import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
import oracle
from gpu_helpers import DEV, ITERATE_TOL, R_FP16, R_FP32, evd, rel_err, residual, to_dev, to_host

pytestmark = pytest.mark.gpu

EIG_TOL = 2e-5  # relative to the largest eigenvalue


def gram_stack(N, B, seed, eps=1e-3):
    """A_i = G_i G_i^T / (2B) + eps I, G_i in R^{B x 2B} iid N(0,1), built in fp64, rounded once."""
    g = di.rng(seed)
    A = np.empty((N, B, B), dtype=np.float32)
    for i in range(N):
        G = g.standard_normal((B, 2 * B))
        M = G @ G.T / (2 * B) + eps * np.eye(B)
        A[i] = (0.5 * (M + M.T)).astype(np.float32)
    return A


def check_eigs(w, A):
    for b in range(A.shape[0]):
        ref = np.sort(oracle.jacobi_eigh(A[b])[0])
        assert np.max(np.abs(np.sort(w[b]) - ref)) <= EIG_TOL * ref[-1], b


def check_against_oracle(A, X, w, tol=ITERATE_TOL):
    Xh = to_host(X)
    ref = oracle.inverse_root_evd(A)
    assert rel_err(Xh, ref).max() <= tol
    assert residual(Xh, A).max() <= R_FP32
    assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))  # Y Y^T computed on one triangle and mirrored
    check_eigs(to_host(w), A)
    return Xh


@pytest.mark.parametrize("refine", [0, 1])
def test_evd_tiny(refine):
    """4 x 64 x 64 (one pair of column blocks: a sweep is one round, i.e. one scalar cyclic Jacobi
    sweep over the whole block; the last sweep finds nothing to rotate)."""
    A = di.tiny_stack()
    X, w, sweeps, status = evd(to_dev(A), refine=refine)
    assert (to_host(status) == 0).all()
    check_against_oracle(A, X, w)
    sw = to_host(sweeps)
    assert ((sw >= 3) & (sw <= 12 + 4 * refine)).all()


@pytest.mark.parametrize("B", [128, 192, 320])
def test_evd_pair_counts(B):
    """2, 3 and 5 pairs per round (K = 4, 6, 10 column blocks of the circle schedule)."""
    A = gram_stack(3, B, seed=11 + B)
    X, w, sweeps, status = evd(to_dev(A))
    assert (to_host(status) == 0).all()
    check_against_oracle(A, X, w)
    assert (to_host(sweeps) >= 2).all()


def test_evd_conditioned_refined():
    """16 x 256 x 256, kappa 1e4: the refinement pass keeps the residual under the fp32 gate."""
    A = di.conditioned_stack()[0]
    Ad = to_dev(A)
    X, w, sweeps, status = evd(Ad, refine=1)
    assert (to_host(status) == 0).all()
    Xh = to_host(X)
    r1 = residual(Xh, A)
    assert r1.max() <= R_FP32
    X0, _, _, _ = evd(Ad, refine=0)
    assert r1.mean() < residual(to_host(X0), A).mean()
    assert rel_err(Xh, oracle.inverse_root_evd(A)).max() <= 1e-3
    assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))
    check_eigs(to_host(w), A)


def test_evd_diagonal_input():
    """A diagonal block needs no rotation: one sweep, the eigenvalues are the diagonal exactly and
    X = diag(d^{-1/4}) up to the rounding of d^{-1/8} and of its square."""
    g = di.rng(21)
    d = np.exp(g.uniform(np.log(1e-3), 0.0, (2, 192))).astype(np.float32)
    A = np.zeros((2, 192, 192), dtype=np.float32)
    for b in range(2):
        np.fill_diagonal(A[b], d[b])
    X, w, sweeps, status = evd(to_dev(A))
    assert (to_host(status) == 0).all()
    assert (to_host(sweeps) == 1).all()
    assert np.array_equal(to_host(w), d.astype(np.float64))
    Xh = to_host(X)
    for b in range(2):
        assert np.count_nonzero(Xh[b] - np.diag(np.diag(Xh[b]))) == 0
        np.testing.assert_allclose(np.diag(Xh[b]), d[b].astype(np.float64) ** -0.25, rtol=3e-7)


@pytest.mark.parametrize("refine", [0, 1])
def test_evd_scale_equivariance(refine):
    """X(256 A) = X(A) / 4 and w(256 A) = 256 w(A) bitwise: rotations depend on ratios only, the
    products scale exactly and w^{-1/8} is three square roots."""
    A = gram_stack(2, 128, seed=31)
    X1, w1, s1, _ = evd(to_dev(A), refine=refine)
    X2, w2, s2, _ = evd(to_dev(256.0 * A), refine=refine)
    assert torch.equal(X2 * 4.0, X1)
    assert torch.equal(w2, 256.0 * w1)
    assert torch.equal(s1, s2)


def test_evd_batch_independence():
    """A block solved alone equals the same block solved inside a stack, bit for bit."""
    A = gram_stack(5, 128, seed=41)
    X, w, sweeps, _ = evd(to_dev(A))
    Xs, ws_, ss, _ = evd(to_dev(A[3:4]))
    assert torch.equal(X[3:4], Xs)
    assert torch.equal(w[3:4], ws_)
    assert int(sweeps[3]) == int(ss[0])


def test_evd_flags_bad_blocks():
    """A block with a negative eigenvalue or a NaN gets status bit 0 and a NaN result; the other
    blocks are unaffected."""
    A = gram_stack(4, 128, seed=51)
    Q = di.haar_orthogonal(di.rng(52), 128)
    lam = np.linspace(-0.5, 1.0, 128)
    A[1] = ((Q * lam[None, :]) @ Q.T).astype(np.float32)
    A[2, 5, 7] = A[2, 7, 5] = np.nan
    X, w, sweeps, status = evd(to_dev(A))
    st = to_host(status).astype(int)
    assert st[1] & 1 and st[2] & 1
    assert st[0] == 0 and st[3] == 0
    Xh = to_host(X)
    assert np.isnan(Xh[1]).all() and np.isnan(Xh[2]).all()
    Xa, _, _, _ = evd(to_dev(A[[0, 3]]))
    assert np.array_equal(Xh[[0, 3]], to_host(Xa))


def test_evd_sweep_limit_flag():
    """max_sweeps = 1 stops a dense block before it converges: status bit 2, one sweep counted."""
    A = gram_stack(2, 256, seed=61)
    X, w, sweeps, status = evd(to_dev(A), max_sweeps=1)
    assert (to_host(status).astype(int) == 4).all()
    assert (to_host(sweeps) == 1).all()


# ---------------------------------------------------------------------------------------------------
# first pass with binary16 operands ([PT] Resultados Experimentais: FP16 for the EVD root)
# ---------------------------------------------------------------------------------------------------

FP16_ITERATE_TOL = 1e-3


def check_fp16(A, X, w, status, sweeps, max_sweeps=20):
    assert (to_host(status) == 0).all()
    Xh = to_host(X)
    r = residual(Xh, A)
    e = rel_err(Xh, oracle.inverse_root_evd(A))
    print("fp16 evd: residual max %.3e, iterate error max %.3e, sweeps %s" % (r.max(), e.max(), to_host(sweeps)))
    assert r.max() <= R_FP16
    assert e.max() <= FP16_ITERATE_TOL
    assert np.array_equal(Xh, np.swapaxes(Xh, 1, 2))
    check_eigs(to_host(w), A)
    assert (to_host(sweeps) <= 2 * max_sweeps).all()
    return Xh


def test_evd_fp16_tiny():
    A = di.tiny_stack()
    X, w, sweeps, status = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    Xh = check_fp16(A, X, w, status, sweeps)
    assert rel_err(Xh, oracle.inverse_root_evd(A)).max() <= ITERATE_TOL
    assert residual(Xh, A).max() <= R_FP32


@pytest.mark.parametrize("B", [128, 192, 320])
def test_evd_fp16_pair_counts(B):
    A = gram_stack(3, B, seed=11 + B)
    X, w, sweeps, status = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    Xh = check_fp16(A, X, w, status, sweeps)
    assert rel_err(Xh, oracle.inverse_root_evd(A)).max() <= ITERATE_TOL
    assert residual(Xh, A).max() <= R_FP32


def test_evd_fp16_conditioned():
    """16 x 256 x 256, kappa 1e4: the binary16 pass leaves the small eigenvalues to the fp32 pass,
    which forms H from the input again; the result stays within the binary16 gate and close to the
    fp32 solve's."""
    A = di.conditioned_stack()[0]
    Ad = to_dev(A)
    X, w, sweeps, status = evd(Ad, refine=1, prec=dash.DASH_FP16)
    Xh = check_fp16(A, X, w, status, sweeps)
    X32, _, _, _ = evd(Ad, refine=1)
    r16, r32 = residual(Xh, A), residual(to_host(X32), A)
    print("kappa 1e4: residual fp16 pass %.3e, fp32 pass %.3e" % (r16.max(), r32.max()))
    assert r16.max() <= max(3 * r32.max(), R_FP32)


def test_evd_fp16_small_scale():
    """Entries around 1e-9 (far below binary16's normal range before the prescale): the per-block
    power-of-two prescale keeps the operands normal."""
    A = (gram_stack(2, 128, seed=71) * np.float32(1e-9)).astype(np.float32)
    X, w, sweeps, status = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    check_fp16(A, X, w, status, sweeps)


def test_evd_fp16_scale_equivariance_and_batch():
    """X(256 A) = X(A) / 4 bitwise (the prescale absorbs a power of two exactly), and a block solved
    alone equals the same block inside a stack."""
    A = gram_stack(3, 128, seed=81)
    X1, w1, s1, _ = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    X2, w2, s2, _ = evd(to_dev(256.0 * A), refine=1, prec=dash.DASH_FP16)
    assert torch.equal(X2 * 4.0, X1)
    assert torch.equal(w2, 256.0 * w1)
    assert torch.equal(s1, s2)
    Xs, ws_, ss, _ = evd(to_dev(A[1:2]), refine=1, prec=dash.DASH_FP16)
    assert torch.equal(X1[1:2], Xs)
    assert int(s1[1]) == int(ss[0])


def test_evd_fp16_flags_bad_blocks():
    """As test_evd_flags_bad_blocks with the binary16 products: a negative eigenvalue and a NaN are
    flagged, and the good blocks equal the same blocks solved alone."""
    A = gram_stack(4, 128, seed=51)
    Q = di.haar_orthogonal(di.rng(52), 128)
    lam = np.linspace(-0.5, 1.0, 128)
    A[1] = ((Q * lam[None, :]) @ Q.T).astype(np.float32)
    A[2, 5, 7] = A[2, 7, 5] = np.nan
    X, w, sweeps, status = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    st = to_host(status).astype(int)
    assert st[1] & 1 and st[2] & 1
    assert st[0] == 0 and st[3] == 0
    Xh = to_host(X)
    assert np.isnan(Xh[1]).all() and np.isnan(Xh[2]).all()
    Xa, _, _, _ = evd(to_dev(A[[0, 3]]), refine=1, prec=dash.DASH_FP16)
    assert np.array_equal(Xh[[0, 3]], to_host(Xa))


def test_evd_fp16_differs_from_fp32_first_pass():
    """The binary16 pass really runs: its result is not bitwise the fp32 solve's."""
    A = gram_stack(2, 128, seed=91)
    X16, _, _, _ = evd(to_dev(A), refine=1, prec=dash.DASH_FP16)
    X32, _, _, _ = evd(to_dev(A), refine=1)
    assert not torch.equal(X16, X32)
