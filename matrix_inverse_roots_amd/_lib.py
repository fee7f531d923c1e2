"""ctypes binding of include/dash.h.  Argument marshalling only; all work runs in libdash.so.

Each ``dash_*`` function mirrors the C call of the same name.  Device buffers are torch tensors
(contiguous, on the GPU); sizes are passed explicitly as in the C ABI.  ``stream=None`` means
torch's current HIP stream on the tensors' device.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdash.so")

DASH_OK, DASH_ERR_INVALID_ARG, DASH_ERR_SHAPE, DASH_ERR_WORKSPACE, DASH_ERR_UNSUPPORTED, DASH_ERR_DEVICE = range(6)
DASH_FP32, DASH_FP16, DASH_BF16, DASH_FP32_SPLIT = 0, 1, 2, 3
DASH_SCALE_FROBENIUS, DASH_SCALE_POWER = 0, 1
DASH_OP_SCALE, DASH_OP_NDB, DASH_OP_CN, DASH_OP_CHEB, DASH_OP_APPLY, DASH_OP_STATS, DASH_OP_EVD = range(7)


class DashError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (call, dash_status_string(status), status))


class DashMat(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libdash.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError("libdash.so is not built; run `python -m matrix_inverse_roots_amd.build`")
        lib = ctypes.CDLL(library_path)
        vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_size_t)
        st = ctypes.c_int
        sig = {
            "dash_stack": (st, [ctypes.POINTER(DashMat), i32, i32, vp, vp]),
            "dash_unstack": (st, [vp, i32, ctypes.POINTER(DashMat), i32, vp]),
            "dash_update_stats": (st, [vp, i64, i32, f32, vp, vp]),
            "dash_update_stats_prec": (st, [vp, i64, i32, f32, st, vp, vp]),
            "dash_scale": (st, [vp, i64, i32, st, st, i32, i32, vp, vp, vp, sz, vp]),
            "dash_inverse_root_ndb": (st, [vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_ndb_prec": (st, [vp, vp, i64, i32, i32, i32, st, vp, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_cn": (st, [vp, vp, i64, i32, i32, i32, st, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_ndb_half": (st, [vp, vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_ndb_lowp": (st, [vp, vp, i64, i32, i32, i32, st, i32, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_ndb_adaptive": (st, [vp, vp, i64, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, sz,
                                                    vp]),
            "dash_inverse_root_cn_adaptive": (st, [vp, vp, i64, i32, i32, i32, f32, st, vp, vp, vp, vp, vp, sz, vp]),
            "dash_inverse_root_cheb": (st, [vp, vp, i64, i32, i32, f64, f64, vp, vp, vp, sz, vp]),
            "dash_inverse_root_cheb_prec": (st, [vp, vp, i64, i32, i32, f64, f64, st, vp, vp, vp, sz, vp]),
            "dash_inverse_root_evd": (st, [vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dash_apply": (st, [vp, vp, vp, i64, i32, vp, vp, sz, vp]),
            "dash_apply_prec": (st, [vp, vp, vp, i64, i32, st, vp, vp, sz, vp]),
            "dash_workspace_size": (st, [st, i64, i32, st, i32, ctypes.POINTER(sz)]),
            "dash_solver_products": (i64, [st, i32, i32]),
            "dash_flops": (f64, [st, i64, i32, st, i32, i32]),
            "dash_status_string": (ctypes.c_char_p, [st]),
            "dash_abi_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Plain integers pass through (tests of the ABI)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    dev = next((t.device for t in tensors if hasattr(t, "device") and t.device.type == "cuda"), None)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(name, status):
    if status != DASH_OK:
        raise DashError(name, status)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dash_status_string(status: int) -> str:
    return library().dash_status_string(status).decode()


def dash_abi_version() -> int:
    return library().dash_abi_version()


def dash_solver_products(op: int, iters1: int, iters2: int = 0) -> int:
    return library().dash_solver_products(op, iters1, iters2)


def dash_flops(op: int, N: int, B: int, prec: int = DASH_FP32, a1: int = 0, a2: int = 0) -> float:
    return library().dash_flops(op, N, B, prec, a1, a2)


def dash_workspace_size(op: int, N: int, B: int, prec: int = DASH_FP32, k_or_degree: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check("dash_workspace_size", library().dash_workspace_size(op, N, B, prec, k_or_degree, ctypes.byref(out)))
    return out.value


def workspace(op: int, N: int, B: int, prec: int = DASH_FP32, k_or_degree: int = 0, device="cuda"):
    """A byte tensor of the size dash_workspace_size reports (None when no workspace is needed)."""
    import torch

    n = dash_workspace_size(op, N, B, prec, k_or_degree)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def _mats(ts):
    arr = (DashMat * len(ts))()
    for i, t in enumerate(ts):
        arr[i].ptr = _ptr(t)
        arr[i].rows, arr[i].cols = t.shape
        arr[i].ld = t.stride(0)
    return arr


def dash_stack(grads, B: int, G_stack, stream=None):
    arr = _mats(grads)
    _check("dash_stack", library().dash_stack(arr, len(grads), B, _ptr(G_stack), _stream(stream, G_stack)))


def dash_unstack(U_stack, B: int, outs, stream=None):
    arr = _mats(outs)
    _check("dash_unstack", library().dash_unstack(_ptr(U_stack), B, arr, len(outs), _stream(stream, U_stack)))


def dash_update_stats(G_stack, NG: int, B: int, beta: float, A, stream=None):
    _check("dash_update_stats",
           library().dash_update_stats(_ptr(G_stack), NG, B, beta, _ptr(A), _stream(stream, A)))


def dash_update_stats_prec(G_stack, NG: int, B: int, beta: float, prec: int, A, stream=None):
    _check("dash_update_stats_prec",
           library().dash_update_stats_prec(_ptr(G_stack), NG, B, beta, prec, _ptr(A), _stream(stream, A)))


def dash_scale(A, N: int, B: int, how: int, prec: int, k: int, steps: int, V0, s, ws=None, stream=None):
    _check("dash_scale", library().dash_scale(_ptr(A), N, B, how, prec, k, steps, _ptr(V0), _ptr(s), _ptr(ws),
                                              _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_ndb(A, s, N: int, B: int, iters1: int, iters2: int, X, sqrt_out=None, monitor=None,
                          status=None, ws=None, stream=None):
    _check("dash_inverse_root_ndb",
           library().dash_inverse_root_ndb(_ptr(A), _ptr(s), N, B, iters1, iters2, _ptr(X), _ptr(sqrt_out),
                                           _ptr(monitor), _ptr(status), _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_ndb_prec(A, s, N: int, B: int, iters1: int, iters2: int, prec: int, X, sqrt_out=None,
                               monitor=None, status=None, ws=None, stream=None):
    _check("dash_inverse_root_ndb_prec",
           library().dash_inverse_root_ndb_prec(_ptr(A), _ptr(s), N, B, iters1, iters2, prec, _ptr(X), _ptr(sqrt_out),
                                                _ptr(monitor), _ptr(status), _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_cn(A, s, N: int, B: int, p: int, iters: int, prec: int, X, monitor=None, status=None,
                         ws=None, stream=None):
    _check("dash_inverse_root_cn",
           library().dash_inverse_root_cn(_ptr(A), _ptr(s), N, B, p, iters, prec, _ptr(X), _ptr(monitor),
                                          _ptr(status), _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_ndb_half(A, s, N: int, B: int, iters1: int, iters2: int, refine: int, X, monitor=None,
                               status=None, ws=None, stream=None):
    _check("dash_inverse_root_ndb_half",
           library().dash_inverse_root_ndb_half(_ptr(A), _ptr(s), N, B, iters1, iters2, refine, _ptr(X),
                                                _ptr(monitor), _ptr(status), _ptr(ws), _nbytes(ws),
                                                _stream(stream, A)))


def dash_inverse_root_ndb_lowp(A, s, N: int, B: int, iters1: int, iters2: int, prec: int, refine: int, X,
                               monitor=None, status=None, ws=None, stream=None):
    _check("dash_inverse_root_ndb_lowp",
           library().dash_inverse_root_ndb_lowp(_ptr(A), _ptr(s), N, B, iters1, iters2, prec, refine, _ptr(X),
                                                _ptr(monitor), _ptr(status), _ptr(ws), _nbytes(ws),
                                                _stream(stream, A)))


def dash_inverse_root_ndb_adaptive(A, s, N: int, B: int, max_iters1: int, max_iters2: int, tol: float, X, monitor,
                                   sqrt_out=None, steps=None, status=None, ws=None, stream=None):
    _check("dash_inverse_root_ndb_adaptive",
           library().dash_inverse_root_ndb_adaptive(_ptr(A), _ptr(s), N, B, max_iters1, max_iters2, tol, _ptr(X),
                                                    _ptr(sqrt_out), _ptr(monitor), _ptr(steps), _ptr(status),
                                                    _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_cn_adaptive(A, s, N: int, B: int, p: int, max_iters: int, tol: float, prec: int, X, monitor,
                                  steps=None, status=None, ws=None, stream=None):
    _check("dash_inverse_root_cn_adaptive",
           library().dash_inverse_root_cn_adaptive(_ptr(A), _ptr(s), N, B, p, max_iters, tol, prec, _ptr(X),
                                                   _ptr(monitor), _ptr(steps), _ptr(status), _ptr(ws), _nbytes(ws),
                                                   _stream(stream, A)))


def dash_inverse_root_cheb(A, s, N: int, B: int, degree: int, lo: float, hi: float, X, status=None, ws=None,
                           stream=None):
    _check("dash_inverse_root_cheb",
           library().dash_inverse_root_cheb(_ptr(A), _ptr(s), N, B, degree, lo, hi, _ptr(X), _ptr(status), _ptr(ws),
                                            _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_cheb_prec(A, s, N: int, B: int, degree: int, lo: float, hi: float, prec: int, X, status=None,
                                ws=None, stream=None):
    _check("dash_inverse_root_cheb_prec",
           library().dash_inverse_root_cheb_prec(_ptr(A), _ptr(s), N, B, degree, lo, hi, prec, _ptr(X), _ptr(status),
                                                 _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_inverse_root_evd(A, N: int, B: int, max_sweeps: int, refine: int, X, eigvals=None, sweeps=None, status=None,
                          ws=None, stream=None):
    _check("dash_inverse_root_evd",
           library().dash_inverse_root_evd(_ptr(A), N, B, max_sweeps, refine, _ptr(X), _ptr(eigvals), _ptr(sweeps),
                                           _ptr(status), _ptr(ws), _nbytes(ws), _stream(stream, A)))


def dash_apply(XL, XR, G_stack, NG: int, B: int, U_stack, ws=None, stream=None):
    _check("dash_apply", library().dash_apply(_ptr(XL), _ptr(XR), _ptr(G_stack), NG, B, _ptr(U_stack), _ptr(ws),
                                              _nbytes(ws), _stream(stream, G_stack)))


def dash_apply_prec(XL, XR, G_stack, NG: int, B: int, prec: int, U_stack, ws=None, stream=None):
    _check("dash_apply_prec",
           library().dash_apply_prec(_ptr(XL), _ptr(XR), _ptr(G_stack), NG, B, prec, _ptr(U_stack), _ptr(ws),
                                     _nbytes(ws), _stream(stream, G_stack)))
