"""Host-side tests of the C ABI (no GPU): the library loads, exports every declared call, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import matrix_inverse_roots_amd as dash
from matrix_inverse_roots_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")

# fake, well aligned device addresses: argument checks run before any use of them
P = 1 << 20
P2 = 2 << 20
P3 = 3 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_call():
    lib = ctypes.CDLL(_lib.library_path)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(dash, n), n  # the binding mirrors every name


def test_version_and_status_strings():
    assert dash.dash_abi_version() == 1
    for code in range(6):
        assert dash.dash_status_string(code)
    assert dash.dash_status_string(99) == "unknown status"


def test_product_counts():
    assert dash.dash_solver_products(dash.DASH_OP_NDB, 6, 6) == 30
    assert dash.dash_solver_products(dash.DASH_OP_NDB, 1, 1) == 1
    assert dash.dash_solver_products(dash.DASH_OP_CN, 5) == 16
    assert dash.dash_solver_products(dash.DASH_OP_CN, 1) == 0
    assert dash.dash_solver_products(dash.DASH_OP_CHEB, 24) == 23
    assert dash.dash_solver_products(dash.DASH_OP_NDB, 0, 3) == -1


def test_workspace_sizes():
    N, B = 16, 256
    stack32 = N * B * B * 4
    assert dash.dash_workspace_size(dash.DASH_OP_NDB, N, B) >= 5 * stack32
    assert dash.dash_workspace_size(dash.DASH_OP_CN, N, B, dash.DASH_FP16) >= 5 * stack32 // 2
    assert dash.dash_workspace_size(dash.DASH_OP_CN, N, B, dash.DASH_FP16) < 5 * stack32
    assert dash.dash_workspace_size(dash.DASH_OP_CHEB, N, B) >= 2 * stack32
    assert dash.dash_workspace_size(dash.DASH_OP_APPLY, N, B) >= stack32
    assert dash.dash_workspace_size(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 0) == 0
    assert dash.dash_workspace_size(dash.DASH_OP_SCALE, N, B, dash.DASH_FP16, 32) > N * B * B * 2
    for bad_B in (0, 32, 100, 8256):
        with pytest.raises(dash.DashError) as ei:
            dash.dash_workspace_size(dash.DASH_OP_NDB, N, bad_B)
        assert ei.value.status == _lib.DASH_ERR_SHAPE
    with pytest.raises(dash.DashError):
        dash.dash_workspace_size(dash.DASH_OP_SCALE, N, B, dash.DASH_FP32, 33)


def _status_of(fn, *args, **kw):
    with pytest.raises(dash.DashError) as ei:
        fn(*args, stream=0, **kw)
    return ei.value.status


class FakeWs:
    """Stands in for a workspace tensor: a pointer and a byte count."""

    def __init__(self, ptr, nbytes):
        self.ptr, self.n = ptr, nbytes

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def test_ndb_argument_errors():
    N, B = 4, 64
    ws = FakeWs(P3, dash.dash_workspace_size(dash.DASH_OP_NDB, N, B))
    f = dash.dash_inverse_root_ndb
    assert _status_of(f, None, P2, N, B, 5, 5, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG      # null A
    assert _status_of(f, P + 4, P2, N, B, 5, 5, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG     # misaligned
    assert _status_of(f, P, P2, N, B, 5, 5, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG         # X aliases A
    assert _status_of(f, P, P2, N, B, 0, 5, P3, ws=ws) == _lib.DASH_ERR_INVALID_ARG        # iters < 1
    assert _status_of(f, P, P2, 0, B, 5, 5, P3, ws=ws) == _lib.DASH_ERR_INVALID_ARG        # N < 1
    assert _status_of(f, P, P2, N, 96, 5, 5, P3, ws=ws) == _lib.DASH_ERR_SHAPE             # B % 64
    small = FakeWs(P3, ws.n - 1)
    assert _status_of(f, P, P2, N, B, 5, 5, 5 * P, ws=small) == _lib.DASH_ERR_WORKSPACE
    assert _status_of(f, P, P2, N, B, 5, 5, 5 * P, ws=FakeWs(P3 + 16, ws.n)) == _lib.DASH_ERR_WORKSPACE


def test_cn_cheb_scale_apply_stats_argument_errors():
    N, B = 4, 64
    ws = FakeWs(P3, 1 << 30)
    assert _status_of(dash.dash_inverse_root_cn, P, P2, N, B, 2, 5, dash.DASH_FP32, 5 * P,
                      ws=ws) == _lib.DASH_ERR_UNSUPPORTED                                   # p != 4
    assert _status_of(dash.dash_inverse_root_cn, P, P2, N, B, 4, 0, dash.DASH_FP32, 5 * P,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_inverse_root_cn, P, P2, N, B, 4, 3, 7, 5 * P,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG                                   # bad precision
    f = dash.dash_inverse_root_cheb
    assert _status_of(f, P, P2, N, B, 0, 0.1, 1.0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, N, B, 65, 0.1, 1.0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, N, B, 8, 0.0, 1.0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, N, B, 8, 1.0, 1.0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, N, B, 8, 0.1, float("inf"), 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    g = dash.dash_scale
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 33, 10, P2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG                                   # k > 32
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 0, 10, P2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 8, 0, P2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 8, 10, P2 + 2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG                                   # V0 misaligned
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 8, 10, None, P3,
                      ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE                         # V0 NULL: seeded
    assert _status_of(g, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32, 8, 10, P2, P3,
                      ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE
    assert _status_of(g, P, N, B, 5, dash.DASH_FP32, 8, 10, P2, P3, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    a = dash.dash_apply
    assert _status_of(a, P, P2, P3, N, B, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG            # U aliases XL
    assert _status_of(a, P, P2, P3, N, B, 5 * P, ws=FakeWs(8 * P, 10)) == _lib.DASH_ERR_WORKSPACE
    u = dash.dash_update_stats
    assert _status_of(u, P, N, B, 1.5, P2) == _lib.DASH_ERR_INVALID_ARG                     # beta > 1
    assert _status_of(u, P, N, B, float("nan"), P2) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(u, P, N, 48, 0.9, P2) == _lib.DASH_ERR_SHAPE


class FakeMat:
    def __init__(self, ptr, rows, cols, ld=None):
        self.ptr, self.shape, self._ld = ptr, (rows, cols), ld if ld is not None else cols

    def data_ptr(self):
        return self.ptr

    def stride(self, d):
        return self._ld if d == 0 else 1


def test_stack_argument_errors():
    B = 64
    assert _status_of(dash.dash_stack, [FakeMat(P, 128, 96)], 96, P2) == _lib.DASH_ERR_SHAPE   # B % 64
    assert _status_of(dash.dash_stack, [FakeMat(P, 0, 96)], B, P2) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_stack, [FakeMat(P, 128, 128, ld=64)], B, P2) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_stack, [FakeMat(P + 8, 128, 128)], B, P2) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_stack, [FakeMat(P, 128, 128)], B, None) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_unstack, P2, B, [FakeMat(P, 64, 130, ld=130)]) == _lib.DASH_ERR_INVALID_ARG


def test_evd_argument_errors_and_counts():
    N, B = 4, 64
    ws = FakeWs(P3, dash.dash_workspace_size(dash.DASH_OP_EVD, N, B))
    assert ws.n >= 2 * N * B * B * 4
    f = dash.dash_inverse_root_evd
    assert _status_of(f, None, N, B, 10, 0, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG     # null A
    assert _status_of(f, P, N, B, 10, 0, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG         # X aliases A
    assert _status_of(f, P, N, B, 0, 0, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG         # max_sweeps < 1
    assert _status_of(f, P, N, B, 101, 0, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, N, B, 10, 2, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG        # refine not 0/1
    assert _status_of(f, P, N, 96, 10, 0, P2, ws=ws) == _lib.DASH_ERR_SHAPE
    assert _status_of(f, P, N, B, 10, 0, P2 + 4, ws=ws) == _lib.DASH_ERR_INVALID_ARG    # misaligned X
    assert _status_of(f, P, N, B, 10, 0, P2, ws=FakeWs(P3, ws.n - 1)) == _lib.DASH_ERR_WORKSPACE
    g = dash.dash_inverse_root_evd_prec
    assert _status_of(g, P, N, B, 10, 0, _lib.DASH_FP16, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG  # fp16 needs refine
    for prec in (_lib.DASH_BF16, _lib.DASH_FP32_SPLIT, 7):
        assert _status_of(g, P, N, B, 10, 1, prec, P2, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, N, B, 10, 1, _lib.DASH_FP16, P2, ws=FakeWs(P3, ws.n - 1)) == _lib.DASH_ERR_WORKSPACE
    # flops: one full sweep of updates per round (P(P-1)/2 blocks x 2 products + P * B/64 tiles) + Y Y^T
    Bf, Nf = 256, 3
    Pp = Bf // 64
    per_round = (Pp * (Pp - 1) // 2 * 2 + Pp * (Bf // 64)) * 2 * 64 ** 3
    tri = (Bf // 128) * (Bf // 128 + 1) / 2 / (Bf // 128) ** 2
    expect = 7 * (Bf // 32 - 1) * per_round * Nf + 2 * Bf ** 3 * Nf * tri
    assert dash.dash_flops(dash.DASH_OP_EVD, Nf, Bf, dash.DASH_FP32, 7, 0) == pytest.approx(expect)
    assert dash.dash_flops(dash.DASH_OP_EVD, Nf, Bf, dash.DASH_FP32, 0, 0) == -1.0


def test_adaptive_argument_errors():
    N, B = 4, 64
    ws = FakeWs(P3, 1 << 30)
    f = dash.dash_inverse_root_ndb_adaptive
    assert _status_of(f, P, P2, N, B, 8, 8, 1e-5, 5 * P, None, ws=ws) == _lib.DASH_ERR_INVALID_ARG    # no monitor
    assert _status_of(f, P, P2, N, B, 8, 8, -1.0, 5 * P, 6 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG   # tol < 0
    assert _status_of(f, P, P2, N, B, 8, 8, float("nan"), 5 * P, 6 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, N, B, 0, 8, 1e-5, 5 * P, 6 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG   # max1 < 1
    assert _status_of(f, P, P2, N, B, 8, 8, 1e-5, 5 * P, 6 * P,
                      ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE
    g = dash.dash_inverse_root_cn_adaptive
    assert _status_of(g, P, P2, N, B, 4, 8, 1e-5, dash.DASH_FP32, 5 * P, None, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, P2, N, B, 4, 8, 1e-5, 7, 5 * P, 6 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG  # bad prec
    assert _status_of(g, P, P2, N, B, 3, 8, 1e-5, dash.DASH_FP32, 5 * P, 6 * P,
                      ws=ws) == _lib.DASH_ERR_UNSUPPORTED                                          # p != 4


def test_bfloat16_queries_and_argument_errors():
    """bfloat16 operands: the half-precision solvers' queries match binary16 (same 2-byte stacks, same
    tile counts); power-iteration scaling and other precisions are refused before any launch."""
    N, B = 16, 256
    for op in (dash.DASH_OP_CN, dash.DASH_OP_NDB):
        assert (dash.dash_workspace_size(op, N, B, dash.DASH_BF16)
                == dash.dash_workspace_size(op, N, B, dash.DASH_FP16))
    assert (dash.dash_flops(dash.DASH_OP_CN, N, B, dash.DASH_BF16, 5, 0)
            == dash.dash_flops(dash.DASH_OP_CN, N, B, dash.DASH_FP16, 5, 0))
    with pytest.raises(dash.DashError) as ei:
        dash.dash_workspace_size(dash.DASH_OP_SCALE, N, B, dash.DASH_BF16, 32)
    assert ei.value.status == _lib.DASH_ERR_UNSUPPORTED
    assert _status_of(dash.dash_scale, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_BF16, 32, 10, P2, P3,
                      ws=FakeWs(4 * P, 1 << 30)) == _lib.DASH_ERR_UNSUPPORTED
    ws = FakeWs(P3, dash.dash_workspace_size(dash.DASH_OP_NDB, 4, 64, dash.DASH_BF16))
    f = dash.dash_inverse_root_ndb_lowp
    assert _status_of(f, P, P2, 4, 64, 6, 6, dash.DASH_FP32, 0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, 4, 64, 6, 6, 7, 0, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(f, P, P2, 4, 64, 6, 6, dash.DASH_BF16, 17, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert (_status_of(f, P, P2, 4, 64, 6, 6, dash.DASH_BF16, 0, 5 * P, ws=FakeWs(P3, ws.n - 1))
            == _lib.DASH_ERR_WORKSPACE)
    assert _status_of(dash.dash_inverse_root_cn, P, P2, 4, 64, 4, 5, 7, 5 * P,
                      ws=FakeWs(P3, 1 << 30)) == _lib.DASH_ERR_INVALID_ARG

def test_split_precision_queries_and_argument_errors():
    """DASH_FP32_SPLIT: the workspace of the fp32 solves; dash_flops counts the Chebyshev products on
    256-wide tiles (fp32 tiles when B % 256 != 0 or at degree 2) and NDB's full products as fp32's; only the *_prec solver entries take it, and they take nothing
    else but DASH_FP32."""
    for B in (256, 320, 1024):
        assert dash.dash_workspace_size(dash.DASH_OP_CHEB, 8, B, dash.DASH_FP32_SPLIT) == \
            dash.dash_workspace_size(dash.DASH_OP_CHEB, 8, B, dash.DASH_FP32)
    full = 2.0 * 1024 ** 3 * 3
    f = dash.dash_flops(dash.DASH_OP_CHEB, 3, 1024, dash.DASH_FP32_SPLIT, 24, 0)
    assert f == pytest.approx(full * 23 * 10 / 16, rel=1e-12)
    assert dash.dash_flops(dash.DASH_OP_CHEB, 3, 1024, dash.DASH_FP32_SPLIT, 2, 0) == \
        dash.dash_flops(dash.DASH_OP_CHEB, 3, 1024, dash.DASH_FP32, 2, 0)  # degree 2: the fp32 cores
    assert dash.dash_flops(dash.DASH_OP_CHEB, 3, 1024, dash.DASH_FP32, 24, 0) == pytest.approx(full * 23 * 36 / 64)
    assert dash.dash_flops(dash.DASH_OP_CHEB, 3, 320, dash.DASH_FP32_SPLIT, 24, 0) == \
        dash.dash_flops(dash.DASH_OP_CHEB, 3, 320, dash.DASH_FP32, 24, 0)
    N, B = 4, 256
    ws = FakeWs(P3, 1 << 30)
    g = dash.dash_inverse_root_cheb_prec
    for prec in (dash.DASH_FP16, dash.DASH_BF16, 7):
        assert _status_of(g, P, P2, N, B, 8, 0.1, 1.0, prec, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, P2, N, B, 0, 0.1, 1.0, dash.DASH_FP32_SPLIT, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(g, P, P2, N, 96, 8, 0.1, 1.0, dash.DASH_FP32_SPLIT, 5 * P, ws=ws) == _lib.DASH_ERR_SHAPE
    assert _status_of(g, P, P2, N, B, 8, 0.1, 1.0, dash.DASH_FP32_SPLIT, 5 * P,
                      ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE
    assert _status_of(dash.dash_inverse_root_cn, P, P2, N, B, 2, 3, dash.DASH_FP32_SPLIT, 5 * P,
                      ws=ws) == _lib.DASH_ERR_UNSUPPORTED                                   # p != 4
    assert dash.dash_workspace_size(dash.DASH_OP_CN, 8, B, dash.DASH_FP32_SPLIT) == \
        dash.dash_workspace_size(dash.DASH_OP_CN, 8, B, dash.DASH_FP32)
    h = dash.dash_inverse_root_ndb_prec
    for prec in (dash.DASH_FP16, dash.DASH_BF16, 7):
        assert _status_of(h, P, P2, N, B, 5, 5, prec, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(h, P, P2, N, B, 0, 5, dash.DASH_FP32_SPLIT, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(h, P, P2, N, 96, 5, 5, dash.DASH_FP32_SPLIT, 5 * P, ws=ws) == _lib.DASH_ERR_SHAPE
    assert _status_of(h, P, P2, N, B, 5, 5, dash.DASH_FP32_SPLIT, 5 * P,
                      ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE
    assert dash.dash_flops(dash.DASH_OP_NDB, 3, 1024, dash.DASH_FP32_SPLIT, 6, 6) == \
        dash.dash_flops(dash.DASH_OP_NDB, 3, 1024, dash.DASH_FP32, 6, 6)
    for prec in (dash.DASH_FP16, dash.DASH_BF16, 7):
        assert _status_of(dash.dash_update_stats_prec, P, N, B, 0.9, prec, P2) == _lib.DASH_ERR_INVALID_ARG
        assert _status_of(dash.dash_apply_prec, P, P2, P3, N, B, prec, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_update_stats_prec, P, N, B, 1.5, dash.DASH_FP32_SPLIT, P2) == \
        _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_apply_prec, P, P2, P3, N, B, dash.DASH_FP32_SPLIT, P, ws=ws) == \
        _lib.DASH_ERR_INVALID_ARG                                                           # U aliases XL
    # the scale takes split products (past the precision check, a short workspace is what stops it)
    assert _status_of(dash.dash_scale, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_FP32_SPLIT, 8, 10, P2, P3,
                      ws=FakeWs(4 * P, 256)) == _lib.DASH_ERR_WORKSPACE
    assert _status_of(dash.dash_scale, P, N, B, dash.DASH_SCALE_POWER, dash.DASH_BF16, 8, 10, P2, P3,
                      ws=ws) == _lib.DASH_ERR_UNSUPPORTED
    assert _status_of(dash.dash_scale, P, N, B, dash.DASH_SCALE_POWER, 7, 8, 10, P2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG


def test_start_pool_generator_matches_splitmix64_definition():
    """dash_inputs.start_pool_counter (the host twin of the library's seeded start pool) against
    SplitMix64 written out with Python integers from its published definition."""
    import dash_inputs as di

    M = (1 << 64) - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    for seed in (0, 7, (1 << 64) - 5):
        pool = di.start_pool_counter(64, 3, seed)
        for e in (0, 1, 2, 100, 191):
            u = sum(mix((seed + (3 * e + q) * 0x9E3779B97F4A7C15) & M) >> 42 for q in (1, 2, 3))
            assert float(pool.reshape(-1)[e]) == (u - 6291456) * 2.0 ** -22
    assert abs(float(di.start_pool_counter(256, 32, 7).mean())) < 0.05


def test_binding_rejects_host_tensors():
    """The binding checks tensor arguments before any pointer reaches the library: a host tensor is
    refused with ValueError (no GPU needed)."""
    import torch

    A = torch.zeros((2, 64, 64))
    s = torch.zeros(2)
    with pytest.raises(ValueError, match="GPU tensor"):
        dash.dash_inverse_root_ndb(A, s, 2, 64, 3, 3, torch.zeros_like(A))
    with pytest.raises(ValueError, match="GPU tensor"):
        dash.dash_scale(A, 2, 64, dash.DASH_SCALE_FROBENIUS, dash.DASH_FP32, 0, 0, None, s, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        dash.dash_stack([torch.zeros((64, 64))], 64, P)


def test_split16_precision_queries_and_argument_errors():
    """DASH_FP32_SPLIT16 (two-piece binary16 products): the Chebyshev solves and NDB take it, the
    Chebyshev solve with the workspace of the fp32 solve and DASH_FP32_SPLIT's flop count; the apply
    takes it with the workspace every prec uses; the statistics take it through dash_update_stats_ws
    (a bound per tile in the workspace); CN, dash_update_stats_prec and the scale reject it."""
    for B in (256, 320, 1024):
        assert dash.dash_workspace_size(dash.DASH_OP_CHEB, 8, B, dash.DASH_FP32_SPLIT16) == \
            dash.dash_workspace_size(dash.DASH_OP_CHEB, 8, B, dash.DASH_FP32)
        for d in (2, 24):
            assert dash.dash_flops(dash.DASH_OP_CHEB, 3, B, dash.DASH_FP32_SPLIT16, d, 0) == \
                dash.dash_flops(dash.DASH_OP_CHEB, 3, B, dash.DASH_FP32_SPLIT, d, 0)
    N, B = 4, 256
    ws = FakeWs(P3, 1 << 30)
    S16 = dash.DASH_FP32_SPLIT16
    g = dash.dash_inverse_root_cheb_prec
    assert _status_of(g, P, P2, N, B, 0, 0.1, 1.0, S16, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG  # degree 0
    assert _status_of(g, P, P2, N, 96, 8, 0.1, 1.0, S16, 5 * P, ws=ws) == _lib.DASH_ERR_SHAPE
    assert _status_of(g, P, P2, N, B, 8, 0.1, 1.0, S16, 5 * P, ws=FakeWs(P3, 16)) == _lib.DASH_ERR_WORKSPACE
    # the workspace holds the magnitude bounds too: one byte short is refused
    need = dash.dash_workspace_size(dash.DASH_OP_CHEB, N, B, S16)
    assert _status_of(g, P, P2, N, B, 8, 0.1, 1.0, S16, 5 * P, ws=FakeWs(P3, need - 1)) == _lib.DASH_ERR_WORKSPACE
    # NDB takes it too (past the precision check, a short workspace is what stops it)
    assert _status_of(dash.dash_inverse_root_ndb_prec, P, P2, N, B, 5, 5, S16, 5 * P, ws=FakeWs(P3, 16)) == \
        _lib.DASH_ERR_WORKSPACE
    assert _status_of(dash.dash_inverse_root_ndb_prec, P, P2, N, B, 0, 5, S16, 5 * P, ws=ws) == \
        _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_inverse_root_cn, P, P2, N, B, 4, 5, S16, 5 * P, ws=ws) == _lib.DASH_ERR_INVALID_ARG
    assert _status_of(dash.dash_update_stats_prec, P, N, B, 0.9, S16, P2) == _lib.DASH_ERR_INVALID_ARG
    need = dash.dash_workspace_size(dash.DASH_OP_STATS, N, B, S16)
    assert need >= 4 * N and need % 256 == 0
    assert dash.dash_workspace_size(dash.DASH_OP_STATS, N, B, dash.DASH_FP32) == 0
    w = dash.dash_update_stats_ws
    assert _status_of(w, P, N, B, 0.9, S16, P2, ws=FakeWs(P3, need - 1)) == _lib.DASH_ERR_WORKSPACE
    assert _status_of(w, P, N, B, 1.5, S16, P2, ws=FakeWs(P3, need)) == _lib.DASH_ERR_INVALID_ARG  # beta
    assert _status_of(w, P, N, 96, 0.9, S16, P2, ws=FakeWs(P3, need)) == _lib.DASH_ERR_SHAPE
    for prec in (dash.DASH_FP16, dash.DASH_BF16, 7):   # other precs: dash_update_stats_prec's answers
        assert _status_of(w, P, N, B, 0.9, prec, P2) == _lib.DASH_ERR_INVALID_ARG
    need = dash.dash_workspace_size(dash.DASH_OP_APPLY, N, B, S16)
    assert need == dash.dash_workspace_size(dash.DASH_OP_APPLY, N, B, dash.DASH_FP32)
    assert need > N * B * B * 4  # the intermediate and the bounds
    assert _status_of(dash.dash_apply_prec, P, P2, P3, N, B, S16, 5 * P, ws=FakeWs(P3, need - 1)) == \
        _lib.DASH_ERR_WORKSPACE
    assert _status_of(dash.dash_apply_prec, P, P2, P3, N, B, S16, P, ws=ws) == _lib.DASH_ERR_INVALID_ARG  # U aliases XL
    assert _status_of(dash.dash_scale, P, N, B, dash.DASH_SCALE_POWER, S16, 8, 10, P2, P3,
                      ws=ws) == _lib.DASH_ERR_INVALID_ARG
