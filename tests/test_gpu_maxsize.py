"""GPU checks at the largest block the ABI takes, B = 8192 (one 256 MiB block), where the fp64 oracle
is too slow to run: properties that hold at any size.  The residual ||X^4 A - I||_F / sqrt(B) of
every solver is evaluated in fp64 with torch products on the device; the scale estimates are
checked against bounds and against each other."""
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
from gpu_helpers import DEV, R_FP16, R_FP32, cheb, cn, frob_scale, ndb, power_scale

pytestmark = pytest.mark.gpu

B = 8192
SHIFT = 1.0  # A = G G^T / B + I: spectrum in about [1, 5] (kappa 5, like the Gram stacks)


@pytest.fixture(scope="module")
def block():
    G = di.gaussian_torch((B, B), seed=41, device=DEV).double()
    A64 = G @ G.T.contiguous() / B + SHIFT * torch.eye(B, device=DEV, dtype=torch.float64)
    A64 = 0.5 * (A64 + A64.T.contiguous())
    del G
    A = A64.float().reshape(1, B, B).contiguous()
    A64 = A.double()[0]
    V0 = torch.from_numpy(di.start_vectors(B, 32)).to(DEV)
    yield A, A64, V0
    del A, A64
    torch.cuda.empty_cache()


def residual64(X, A64):
    x = X[0].double()
    x2 = x @ x
    r = x2 @ x2 @ A64
    r.diagonal().sub_(1.0)
    return float(torch.linalg.matrix_norm(r) / B ** 0.5)


def test_maxsize_scales(block):
    A, A64, V0 = block
    fro = float(torch.linalg.matrix_norm(A64))
    assert abs(float(frob_scale(A)[0]) - fro) <= 1e-6 * fro
    s10 = float(power_scale(A, V0, 10)[0])
    s3 = float(power_scale(A, V0, 3)[0])
    s16 = float(power_scale(A, V0, 10, dash.DASH_FP16)[0])
    s_split = float(power_scale(A, V0, 10, dash.DASH_FP32_SPLIT)[0])
    assert s3 * (1 - 1e-6) <= s10 <= fro          # Rayleigh quotients grow with the steps, below ||A||_2
    assert s10 > 0.85 * (4 + SHIFT)                 # approaches the Marchenko-Pastur edge 4 + SHIFT
    assert abs(s16 - s10) <= 2e-3 * s10
    assert abs(s_split - s10) <= 2e-6 * s10         # split products: an fp32 product


def test_maxsize_ndb(block):
    A, A64, V0 = block
    s = power_scale(A, V0, 10)
    X, R, _, status = ndb(A, s, 8, 8, want_sqrt=True)
    assert int(status[0]) == 0
    assert residual64(X, A64) < R_FP32
    r = R[0].double()
    assert float(torch.linalg.matrix_norm(r @ r - A64) / torch.linalg.matrix_norm(A64)) < 1e-4


@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP16])
def test_maxsize_cn(block, prec):
    A, A64, V0 = block
    s = power_scale(A, V0, 10, prec)
    X, _, status = cn(A, s, 8, prec)
    assert int(status[0]) == 0
    assert residual64(X, A64) < (R_FP32 if prec == dash.DASH_FP32 else R_FP16)
    if prec == dash.DASH_FP16:  # mirrored products: exactly symmetric
        assert torch.equal(X[0], X[0].T)


def test_maxsize_cheb(block):
    A, A64, V0 = block
    s = power_scale(A, V0, 10)
    lo = 0.9 * SHIFT / float(s[0])
    X, status = cheb(A, s, 24, lo, 1.25)
    assert int(status[0]) == 0
    assert residual64(X, A64) < R_FP32
    assert torch.equal(X[0], X[0].T)


def test_maxsize_split_products(block):
    """Split products at B = 8192, where the column gathers' 32-bit byte offsets into a 256 MiB block
    are largest: the Chebyshev solve (every product, the first with A read by columns) and NDB
    (general products, columns gathered) meet the fp32 residual gate and agree with the fp32
    matrix cores' results to well within the iterate tolerance."""
    A, A64, V0 = block
    s = power_scale(A, V0, 10)
    lo = 0.9 * SHIFT / float(s[0])
    X, status = cheb(A, s, 24, lo, 1.25)
    Xs = torch.empty_like(A)
    st = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, 1, B, dash.DASH_FP32_SPLIT, device=DEV)
    dash.dash_inverse_root_cheb_prec(A, s, 1, B, 24, lo, 1.25, dash.DASH_FP32_SPLIT, Xs, status=st, ws=ws)
    del ws
    assert int(st[0]) == 0
    assert residual64(Xs, A64) < R_FP32
    assert torch.equal(Xs[0], Xs[0].T)
    assert float(torch.linalg.matrix_norm(Xs[0].double() - X[0].double()) /
                 torch.linalg.matrix_norm(X[0].double())) < 1e-5
    Xn = torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_NDB, 1, B, dash.DASH_FP32_SPLIT, device=DEV)
    dash.dash_inverse_root_ndb_prec(A, s, 1, B, 8, 8, dash.DASH_FP32_SPLIT, Xn, status=st, ws=ws)
    del ws
    assert int(st[0]) == 0
    assert residual64(Xn, A64) < R_FP32


def test_maxsize_split16_products(block):
    """Two-piece binary16 products at B = 8192, where the magnitude bounds are longest (4224 per-wave
    maxima per block for the Chebyshev launches, 8192 for NDB's iterates and the apply's
    intermediate) and the buffer-addressed epilogue's byte offsets reach 256 MiB: the Chebyshev solve
    and NDB meet the fp32 residual gate and agree with the fp32 matrix cores' results within 1e-5,
    and so does the apply X_cheb A X_ndb."""
    A, A64, V0 = block
    S16 = dash.DASH_FP32_SPLIT16
    s = power_scale(A, V0, 10)
    lo = 0.9 * SHIFT / float(s[0])
    st = torch.empty(1, dtype=torch.int32, device=DEV)

    def rel(P, Q):
        return float(torch.linalg.matrix_norm(P[0].double() - Q[0].double()) / torch.linalg.matrix_norm(Q[0].double()))

    X, _ = cheb(A, s, 24, lo, 1.25)
    Xs = torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_CHEB, 1, B, S16, device=DEV)
    dash.dash_inverse_root_cheb_prec(A, s, 1, B, 24, lo, 1.25, S16, Xs, status=st, ws=ws)
    del ws
    assert int(st[0]) == 0
    assert residual64(Xs, A64) < R_FP32
    assert torch.equal(Xs[0], Xs[0].T)
    print("cheb split16 vs fp32", rel(Xs, X))
    assert rel(Xs, X) < 1e-5
    del X
    Xn = torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_NDB, 1, B, S16, device=DEV)
    dash.dash_inverse_root_ndb_prec(A, s, 1, B, 8, 8, S16, Xn, status=st, ws=ws)
    del ws
    assert int(st[0]) == 0
    assert residual64(Xn, A64) < R_FP32
    U16, U32 = torch.empty_like(A), torch.empty_like(A)
    ws = dash.workspace(dash.DASH_OP_APPLY, 1, B, S16, device=DEV)
    dash.dash_apply_prec(Xs, Xn, A, 1, B, S16, U16, ws)
    dash.dash_apply_prec(Xs, Xn, A, 1, B, dash.DASH_FP32, U32, ws)
    del ws
    print("apply split16 vs fp32", rel(U16, U32))
    assert rel(U16, U32) < 1e-5


def test_maxsize_split16_statistics(block):
    """dash_update_stats_ws with two-piece binary16 products at B = 8192 (G G^T reading G's rows,
    G^T G gathering its columns at the largest byte offsets): L and R agree with the fp32 matrix
    cores' update within 1e-5 and are exactly symmetric."""
    A, _, _ = block
    G = di.gaussian_torch((1, B, B), seed=43, device=DEV, std=1e-3)
    S0 = torch.cat([A, A]) * 1e-3
    S16, S32 = S0.clone(), S0.clone()
    ws = dash.workspace(dash.DASH_OP_STATS, 1, B, dash.DASH_FP32_SPLIT16, device=DEV)
    dash.dash_update_stats_ws(G, 1, B, 0.95, dash.DASH_FP32_SPLIT16, S16, ws)
    dash.dash_update_stats_prec(G, 1, B, 0.95, dash.DASH_FP32, S32)
    for i in range(2):
        d = float(torch.linalg.matrix_norm(S16[i].double() - S32[i].double()) / torch.linalg.matrix_norm(S32[i].double()))
        print("stats block", i, "split16 vs fp32", d)
        assert d < 1e-5
        assert torch.equal(S16[i], S16[i].T)
