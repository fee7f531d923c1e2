"""dash_scale_noalloc (the scale with the library's own scratch, for callers that cannot allocate)
against dash_scale: two calls in a row, the second with a smaller input, each equal to the
workspace call bit for bit (the same kernels on the same data); requests beyond the scratch are
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import dash_inputs as di
import matrix_inverse_roots_amd as dash
from matrix_inverse_roots_amd import _lib


def test_noalloc_refuses_requests_beyond_its_scratch():
    lib = dash.library()
    P = 1 << 20
    # 489 fp32 blocks of 1024 need more than the 128 MiB scratch; refused on the host, no launch
    assert lib.dash_scale_noalloc(P, 489, 1024, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, 2 * P, 0, 3 * P,
                                  None) == _lib.DASH_ERR_WORKSPACE
    assert lib.dash_scale_noalloc(P, 57, 1024, dash.DASH_SCALE_POWER, dash.DASH_FP16, 32, 10, 2 * P, 0, 3 * P,
                                  None) == _lib.DASH_ERR_WORKSPACE
    assert lib.dash_scale_noalloc(P, 4, 1024, dash.DASH_SCALE_POWER, dash.DASH_FP32, 33, 10, 2 * P, 0, 3 * P,
                                  None) == _lib.DASH_ERR_INVALID_ARG
    assert lib.dash_scale_noalloc(P, 4, 96, dash.DASH_SCALE_POWER, dash.DASH_FP32, 32, 10, 2 * P, 0, 3 * P,
                                  None) == _lib.DASH_ERR_SHAPE
    assert dash.dash_noalloc_scratch_bytes() == 128 << 20


def _scale_ws(A, N, B, prec, steps, V0):
    s = torch.empty(N, device="cuda")
    ws = dash.workspace(dash.DASH_OP_SCALE, N, B, prec, V0.shape[1], device="cuda")
    dash.dash_scale(A, N, B, dash.DASH_SCALE_POWER, prec, V0.shape[1], steps, V0, s, ws)
    return s


@pytest.mark.gpu
@pytest.mark.parametrize("prec", [dash.DASH_FP32, dash.DASH_FP16])
def test_noalloc_matches_the_workspace_call(prec):
    dev = torch.device("cuda:0")
    calls = [(488 if prec == dash.DASH_FP32 else 56, 1024), (40, 512)]  # the second call smaller
    for seed, (N, B) in zip((300, 301), calls):
        A = di.gram_stack_torch(N, B, seed=seed, device=dev)
        V0 = torch.from_numpy(di.start_vectors(B, 32, seed=seed)).to(dev)
        s_ref = _scale_ws(A, N, B, prec, 10, V0)
        s = torch.full((N,), -1.0, device=dev)
        dash.dash_scale_noalloc(A, N, B, dash.DASH_SCALE_POWER, prec, 32, 10, V0, s)
        torch.cuda.synchronize()
        assert torch.equal(s, s_ref), (N, B)
        assert bool((s > 0).all())
        del A
    # the Frobenius scale passes straight through
    A = di.gram_stack_torch(8, 256, seed=302, device=dev)
    s1, s2 = torch.empty(8, device=dev), torch.empty(8, device=dev)
    dash.dash_scale(A, 8, 256, dash.DASH_SCALE_FROBENIUS, dash.DASH_FP32, 0, 0, None, s1, None)
    dash.dash_scale_noalloc(A, 8, 256, dash.DASH_SCALE_FROBENIUS, dash.DASH_FP32, 0, 0, None, s2)
    assert torch.equal(s1, s2)
