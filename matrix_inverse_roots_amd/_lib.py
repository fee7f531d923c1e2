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
DASH_FP32, DASH_FP16, DASH_BF16, DASH_FP32_SPLIT, DASH_FP32_SPLIT16 = 0, 1, 2, 3, 4
DASH_SCALE_FROBENIUS, DASH_SCALE_POWER = 0, 1
(DASH_OP_SCALE, DASH_OP_NDB, DASH_OP_CN, DASH_OP_CHEB, DASH_OP_APPLY, DASH_OP_STATS, DASH_OP_EVD,
 DASH_OP_ROUTED) = range(8)


class DashError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (call, dash_status_string(status), status))


class DashMat(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


class DashVec(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("len", ctypes.c_int64)]


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
            "dash_update_stats_ws": (st, [vp, i64, i32, f32, st, vp, vp, sz, vp]),
            "dash_scale": (st, [vp, i64, i32, st, st, i32, i32, vp, ctypes.c_uint64, vp, vp, sz, vp]),
            "dash_start_vectors": (st, [i32, i32, ctypes.c_uint64, vp, vp]),
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
            "dash_inverse_root_evd_prec": (st, [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dash_apply": (st, [vp, vp, vp, i64, i32, vp, vp, sz, vp]),
            "dash_apply_prec": (st, [vp, vp, vp, i64, i32, st, vp, vp, sz, vp]),
            "dash_inverse_root_cheb_blocks": (st, [vp, vp, i64, i32, i32, f64, vp, f32, f64, st, vp, vp, vp, vp, sz,
                                                   vp]),
            "dash_spectrum_min": (st, [vp, vp, i64, i32, f64, i32, i32, vp, vp, vp, sz, vp]),
            "dash_residual_probe": (st, [vp, vp, i64, i32, i32, vp, vp, vp, sz, vp]),
            "dash_inverse_root_routed": (st, [vp, vp, i64, i32, i32, f64, f64, i32, i32, vp, f32, i32, st, vp, vp, vp,
                                              vp, vp, vp, sz, vp]),
            "dash_scale_noalloc": (st, [vp, i64, i32, st, st, i32, i32, vp, ctypes.c_uint64, vp, vp]),
            "dash_noalloc_scratch_bytes": (sz, []),
            "dash_stack_vec": (st, [ctypes.POINTER(DashVec), i32, i32, vp, vp]),
            "dash_unstack_vec": (st, [vp, i32, ctypes.POINTER(DashVec), i32, vp]),
            "dash_update_stats_vec": (st, [vp, i64, i32, f32, vp, vp]),
            "dash_inverse_sqrt_ndb": (st, [vp, vp, i64, i32, i32, st, vp, vp, vp, vp, sz, vp]),
            "dash_apply_vec": (st, [vp, vp, i64, i32, vp, vp]),
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


class _Args:
    """Host-side checks of one call's tensor arguments before their pointers reach the library.

    A torch tensor must be a contiguous GPU tensor of the expected dtype, on the same device as the
    call's other tensors, with at least as many elements as the call touches; a violation raises
    ValueError and nothing is enqueued.  ``None`` is NULL.  Plain integers and objects that only
    expose ``data_ptr()`` pass through unchecked as raw device addresses (the ABI tests use them).
    """

    def __init__(self, call: str):
        self.call = call
        self.device = None

    def _tensor(self, t, name):
        import torch

        if not isinstance(t, torch.Tensor):
            return False
        if t.device.type != "cuda":
            raise ValueError("%s: %s must be a GPU tensor, got one on %s" % (self.call, name, t.device))
        if self.device is None:
            self.device = t.device
        elif t.device != self.device:
            raise ValueError("%s: %s is on %s, the call's other tensors on %s" % (self.call, name, t.device,
                                                                                  self.device))
        return True

    def ptr(self, t, name, dtype="float32", numel=0):
        """Pointer of tensor argument `name` of `dtype` ('float32', 'int32' or None for any) holding
        at least `numel` elements."""
        if t is None:
            return None
        if isinstance(t, int):
            return t
        if self._tensor(t, name):
            import torch

            want = {"float32": torch.float32, "int32": torch.int32}.get(dtype)
            if want is not None and t.dtype != want:
                raise ValueError("%s: %s must be %s, got %s" % (self.call, name, dtype, t.dtype))
            if not t.is_contiguous():
                raise ValueError("%s: %s must be contiguous" % (self.call, name))
            if t.numel() < numel:
                raise ValueError("%s: %s holds %d elements, the call touches %d" % (self.call, name, t.numel(),
                                                                                     int(numel)))
        return t.data_ptr()

    def ws(self, t):
        """Workspace tensor: any dtype, contiguous, on the call's device; its byte size is checked by
        the library against dash_workspace_size."""
        if t is None or isinstance(t, int):
            return t
        if self._tensor(t, "ws") and not t.is_contiguous():
            raise ValueError("%s: ws must be contiguous" % self.call)
        return t.data_ptr()

    def mats(self, ts, name):
        """dash_mat descriptors of 2-D fp32 GPU matrices with unit column stride."""
        arr = (DashMat * len(ts))()
        for i, t in enumerate(ts):
            if self._tensor(t, "%s[%d]" % (name, i)):
                import torch

                if t.dim() != 2 or t.dtype != torch.float32 or t.stride(1) != 1:
                    raise ValueError("%s: %s[%d] must be a 2-D float32 matrix with unit column stride"
                                     % (self.call, name, i))
            arr[i].ptr = t.data_ptr()
            arr[i].rows, arr[i].cols = t.shape
            arr[i].ld = t.stride(0)
        return arr

    def vecs(self, ts, name):
        """dash_vec descriptors of contiguous 1-D fp32 GPU vectors."""
        arr = (DashVec * len(ts))()
        for i, t in enumerate(ts):
            if self._tensor(t, "%s[%d]" % (name, i)):
                import torch

                if t.dim() != 1 or t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("%s: %s[%d] must be a contiguous 1-D float32 vector" % (self.call, name, i))
            arr[i].ptr = t.data_ptr()
            arr[i].len = t.shape[0]
        return arr

    def stream(self, stream):
        if stream is not None:
            return stream if isinstance(stream, int) else stream.cuda_stream
        import torch

        return torch.cuda.current_stream(self.device).cuda_stream


def _check(name, status):
    if status != DASH_OK:
        raise DashError(name, status)


def _nbytes(t):
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _tiles(shapes, B):
    return sum((-(-r // B)) * (-(-c // B)) for r, c in shapes) if B > 0 else 0


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


def dash_stack(grads, B: int, G_stack, stream=None):
    a = _Args("dash_stack")
    arr = a.mats(grads, "grads")
    n = _tiles([tuple(t.shape) for t in grads], B) * B * B
    _check("dash_stack", library().dash_stack(arr, len(grads), B, a.ptr(G_stack, "G_stack", numel=n), a.stream(stream)))


def dash_unstack(U_stack, B: int, outs, stream=None):
    a = _Args("dash_unstack")
    arr = a.mats(outs, "outs")
    n = _tiles([tuple(t.shape) for t in outs], B) * B * B
    _check("dash_unstack", library().dash_unstack(a.ptr(U_stack, "U_stack", numel=n), B, arr, len(outs),
                                                  a.stream(stream)))


def dash_update_stats(G_stack, NG: int, B: int, beta: float, A, stream=None):
    a = _Args("dash_update_stats")
    _check("dash_update_stats",
           library().dash_update_stats(a.ptr(G_stack, "G_stack", numel=NG * B * B), NG, B, beta,
                                       a.ptr(A, "A", numel=2 * NG * B * B), a.stream(stream)))


def dash_update_stats_prec(G_stack, NG: int, B: int, beta: float, prec: int, A, stream=None):
    a = _Args("dash_update_stats_prec")
    _check("dash_update_stats_prec",
           library().dash_update_stats_prec(a.ptr(G_stack, "G_stack", numel=NG * B * B), NG, B, beta, prec,
                                            a.ptr(A, "A", numel=2 * NG * B * B), a.stream(stream)))


def dash_update_stats_ws(G_stack, NG: int, B: int, beta: float, prec: int, A, ws=None, stream=None):
    a = _Args("dash_update_stats_ws")
    _check("dash_update_stats_ws",
           library().dash_update_stats_ws(a.ptr(G_stack, "G_stack", numel=NG * B * B), NG, B, beta, prec,
                                          a.ptr(A, "A", numel=2 * NG * B * B), a.ws(ws), _nbytes(ws),
                                          a.stream(stream)))


def dash_scale(A, N: int, B: int, how: int, prec: int, k: int, steps: int, V0, s, ws=None, stream=None, seed: int = 0):
    """V0 None with power iteration: the start pool drawn on the device from seed."""
    a = _Args("dash_scale")
    vn = B * k if how == DASH_SCALE_POWER else 0
    _check("dash_scale", library().dash_scale(a.ptr(A, "A", numel=N * B * B), N, B, how, prec, k, steps,
                                              a.ptr(V0, "V0", numel=vn), seed, a.ptr(s, "s", numel=N), a.ws(ws),
                                              _nbytes(ws), a.stream(stream)))


def dash_start_vectors(B: int, k: int, seed: int, V0, stream=None):
    a = _Args("dash_start_vectors")
    _check("dash_start_vectors", library().dash_start_vectors(B, k, seed, a.ptr(V0, "V0", numel=B * k),
                                                              a.stream(stream)))


def dash_scale_noalloc(A, N: int, B: int, how: int, prec: int, k: int, steps: int, V0, s, stream=None,
                       seed: int = 0):
    """dash_scale with the library's own scratch: no workspace argument, nothing allocated."""
    a = _Args("dash_scale_noalloc")
    vn = B * k if how == DASH_SCALE_POWER else 0
    _check("dash_scale_noalloc",
           library().dash_scale_noalloc(a.ptr(A, "A", numel=N * B * B), N, B, how, prec, k, steps,
                                        a.ptr(V0, "V0", numel=vn), seed, a.ptr(s, "s", numel=N),
                                        a.stream(stream)))


def dash_noalloc_scratch_bytes() -> int:
    return library().dash_noalloc_scratch_bytes()


def dash_spectrum_min(A, s, N: int, B: int, hi: float, k: int, steps: int, V0, lam_min, ws=None, stream=None):
    a = _Args("dash_spectrum_min")
    _check("dash_spectrum_min",
           library().dash_spectrum_min(a.ptr(A, "A", numel=N * B * B), a.ptr(s, "s", numel=N), N, B, hi, k, steps,
                                       a.ptr(V0, "V0", numel=B * k), a.ptr(lam_min, "lam_min", numel=N), a.ws(ws),
                                       _nbytes(ws), a.stream(stream)))


def dash_residual_probe(A, X, N: int, B: int, k: int, V0, r, ws=None, stream=None):
    a = _Args("dash_residual_probe")
    _check("dash_residual_probe",
           library().dash_residual_probe(a.ptr(A, "A", numel=N * B * B), a.ptr(X, "X", numel=N * B * B), N, B, k,
                                         a.ptr(V0, "V0", numel=B * k), a.ptr(r, "r", numel=N), a.ws(ws),
                                         _nbytes(ws), a.stream(stream)))


def _solver_ptrs(a, A, s, X, N, B):
    return a.ptr(A, "A", numel=N * B * B), a.ptr(s, "s", numel=N), a.ptr(X, "X", numel=N * B * B)


def dash_inverse_root_ndb(A, s, N: int, B: int, iters1: int, iters2: int, X, sqrt_out=None, monitor=None,
                          status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_ndb")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_ndb",
           library().dash_inverse_root_ndb(pA, ps, N, B, iters1, iters2, pX, a.ptr(sqrt_out, "sqrt_out", numel=N * B * B),
                                           a.ptr(monitor, "monitor", numel=N * (iters1 + iters2)),
                                           a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                           a.stream(stream)))


def dash_inverse_root_ndb_prec(A, s, N: int, B: int, iters1: int, iters2: int, prec: int, X, sqrt_out=None,
                               monitor=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_ndb_prec")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_ndb_prec",
           library().dash_inverse_root_ndb_prec(pA, ps, N, B, iters1, iters2, prec, pX,
                                                a.ptr(sqrt_out, "sqrt_out", numel=N * B * B),
                                                a.ptr(monitor, "monitor", numel=N * (iters1 + iters2)),
                                                a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                a.stream(stream)))


def dash_inverse_root_cn(A, s, N: int, B: int, p: int, iters: int, prec: int, X, monitor=None, status=None,
                         ws=None, stream=None):
    a = _Args("dash_inverse_root_cn")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_cn",
           library().dash_inverse_root_cn(pA, ps, N, B, p, iters, prec, pX, a.ptr(monitor, "monitor", numel=N * iters),
                                          a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                          a.stream(stream)))


def dash_inverse_root_ndb_half(A, s, N: int, B: int, iters1: int, iters2: int, refine: int, X, monitor=None,
                               status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_ndb_half")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_ndb_half",
           library().dash_inverse_root_ndb_half(pA, ps, N, B, iters1, iters2, refine, pX,
                                                a.ptr(monitor, "monitor", numel=N * (iters1 + iters2)),
                                                a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                a.stream(stream)))


def dash_inverse_root_ndb_lowp(A, s, N: int, B: int, iters1: int, iters2: int, prec: int, refine: int, X,
                               monitor=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_ndb_lowp")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_ndb_lowp",
           library().dash_inverse_root_ndb_lowp(pA, ps, N, B, iters1, iters2, prec, refine, pX,
                                                a.ptr(monitor, "monitor", numel=N * (iters1 + iters2)),
                                                a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                a.stream(stream)))


def dash_inverse_root_ndb_adaptive(A, s, N: int, B: int, max_iters1: int, max_iters2: int, tol: float, X, monitor,
                                   sqrt_out=None, steps=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_ndb_adaptive")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_ndb_adaptive",
           library().dash_inverse_root_ndb_adaptive(pA, ps, N, B, max_iters1, max_iters2, tol, pX,
                                                    a.ptr(sqrt_out, "sqrt_out", numel=N * B * B),
                                                    a.ptr(monitor, "monitor", numel=N * (max_iters1 + max_iters2)),
                                                    a.ptr(steps, "steps", "int32", 2 * N),
                                                    a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                    a.stream(stream)))


def dash_inverse_root_cn_adaptive(A, s, N: int, B: int, p: int, max_iters: int, tol: float, prec: int, X, monitor,
                                  steps=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_cn_adaptive")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_cn_adaptive",
           library().dash_inverse_root_cn_adaptive(pA, ps, N, B, p, max_iters, tol, prec, pX,
                                                   a.ptr(monitor, "monitor", numel=N * max_iters),
                                                   a.ptr(steps, "steps", "int32", N),
                                                   a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                   a.stream(stream)))


def dash_inverse_root_cheb(A, s, N: int, B: int, degree: int, lo: float, hi: float, X, status=None, ws=None,
                           stream=None):
    a = _Args("dash_inverse_root_cheb")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_cheb",
           library().dash_inverse_root_cheb(pA, ps, N, B, degree, lo, hi, pX, a.ptr(status, "status", "int32", N),
                                            a.ws(ws), _nbytes(ws), a.stream(stream)))


def dash_inverse_root_cheb_prec(A, s, N: int, B: int, degree: int, lo: float, hi: float, prec: int, X, status=None,
                                ws=None, stream=None):
    a = _Args("dash_inverse_root_cheb_prec")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_cheb_prec",
           library().dash_inverse_root_cheb_prec(pA, ps, N, B, degree, lo, hi, prec, pX,
                                                 a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                 a.stream(stream)))


def dash_inverse_root_cheb_blocks(A, s, N: int, B: int, degree: int, floor: float, lam_min, theta: float, hi: float,
                                  prec: int, X, lo_out=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_cheb_blocks")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_cheb_blocks",
           library().dash_inverse_root_cheb_blocks(pA, ps, N, B, degree, floor, a.ptr(lam_min, "lam_min", numel=N),
                                                   theta, hi, prec, pX, a.ptr(lo_out, "lo_out", numel=N),
                                                   a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                   a.stream(stream)))


def dash_inverse_root_routed(A, s, N: int, B: int, degree: int, floor: float, hi: float, k: int, est_steps: int, V0,
                             tol: float, cn_iters: int, prec: int, X, lam_min=None, resid=None, route=None,
                             status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_routed")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_root_routed",
           library().dash_inverse_root_routed(pA, ps, N, B, degree, floor, hi, k, est_steps,
                                              a.ptr(V0, "V0", numel=B * k), tol, cn_iters, prec, pX,
                                              a.ptr(lam_min, "lam_min", numel=N), a.ptr(resid, "resid", numel=N),
                                              a.ptr(route, "route", "int32", N), a.ptr(status, "status", "int32", N),
                                              a.ws(ws), _nbytes(ws), a.stream(stream)))


def dash_inverse_root_evd(A, N: int, B: int, max_sweeps: int, refine: int, X, eigvals=None, sweeps=None, status=None,
                          ws=None, stream=None):
    a = _Args("dash_inverse_root_evd")
    _check("dash_inverse_root_evd",
           library().dash_inverse_root_evd(a.ptr(A, "A", numel=N * B * B), N, B, max_sweeps, refine,
                                           a.ptr(X, "X", numel=N * B * B), a.ptr(eigvals, "eigvals", numel=N * B),
                                           a.ptr(sweeps, "sweeps", "int32", N), a.ptr(status, "status", "int32", N),
                                           a.ws(ws), _nbytes(ws), a.stream(stream)))


def dash_inverse_root_evd_prec(A, N: int, B: int, max_sweeps: int, refine: int, prec: int, X, eigvals=None,
                               sweeps=None, status=None, ws=None, stream=None):
    a = _Args("dash_inverse_root_evd_prec")
    _check("dash_inverse_root_evd_prec",
           library().dash_inverse_root_evd_prec(a.ptr(A, "A", numel=N * B * B), N, B, max_sweeps, refine, prec,
                                                a.ptr(X, "X", numel=N * B * B),
                                                a.ptr(eigvals, "eigvals", numel=N * B),
                                                a.ptr(sweeps, "sweeps", "int32", N),
                                                a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                                a.stream(stream)))


def dash_apply(XL, XR, G_stack, NG: int, B: int, U_stack, ws=None, stream=None):
    a = _Args("dash_apply")
    n = NG * B * B
    _check("dash_apply", library().dash_apply(a.ptr(XL, "XL", numel=n), a.ptr(XR, "XR", numel=n),
                                              a.ptr(G_stack, "G_stack", numel=n), NG, B,
                                              a.ptr(U_stack, "U_stack", numel=n), a.ws(ws), _nbytes(ws),
                                              a.stream(stream)))


def dash_apply_prec(XL, XR, G_stack, NG: int, B: int, prec: int, U_stack, ws=None, stream=None):
    a = _Args("dash_apply_prec")
    n = NG * B * B
    _check("dash_apply_prec",
           library().dash_apply_prec(a.ptr(XL, "XL", numel=n), a.ptr(XR, "XR", numel=n),
                                     a.ptr(G_stack, "G_stack", numel=n), NG, B, prec,
                                     a.ptr(U_stack, "U_stack", numel=n), a.ws(ws), _nbytes(ws), a.stream(stream)))


def _pieces(lens, B):
    return sum(-(-n // B) for n in lens) if B > 0 else 0


def dash_stack_vec(grads, B: int, g_pieces, stream=None):
    """The pieces of B (the last zero-padded) of 1-D gradients into g_pieces[P, B]."""
    a = _Args("dash_stack_vec")
    arr = a.vecs(grads, "grads")
    n = _pieces([t.shape[0] for t in grads], B) * B
    _check("dash_stack_vec", library().dash_stack_vec(arr, len(grads), B, a.ptr(g_pieces, "g_pieces", numel=n),
                                                      a.stream(stream)))


def dash_unstack_vec(u_pieces, B: int, outs, stream=None):
    a = _Args("dash_unstack_vec")
    arr = a.vecs(outs, "outs")
    n = _pieces([t.shape[0] for t in outs], B) * B
    _check("dash_unstack_vec", library().dash_unstack_vec(a.ptr(u_pieces, "u_pieces", numel=n), B, arr, len(outs),
                                                          a.stream(stream)))


def dash_update_stats_vec(g_pieces, P: int, B: int, beta: float, L, stream=None):
    a = _Args("dash_update_stats_vec")
    _check("dash_update_stats_vec",
           library().dash_update_stats_vec(a.ptr(g_pieces, "g_pieces", numel=P * B), P, B, beta,
                                           a.ptr(L, "L", numel=P * B * B), a.stream(stream)))


def dash_inverse_sqrt_ndb(A, s, N: int, B: int, iters: int, prec: int, X, monitor=None, status=None, ws=None,
                          stream=None):
    a = _Args("dash_inverse_sqrt_ndb")
    pA, ps, pX = _solver_ptrs(a, A, s, X, N, B)
    _check("dash_inverse_sqrt_ndb",
           library().dash_inverse_sqrt_ndb(pA, ps, N, B, iters, prec, pX, a.ptr(monitor, "monitor", numel=N * iters),
                                           a.ptr(status, "status", "int32", N), a.ws(ws), _nbytes(ws),
                                           a.stream(stream)))


def dash_apply_vec(X, g_pieces, P: int, B: int, u_pieces, stream=None):
    a = _Args("dash_apply_vec")
    _check("dash_apply_vec",
           library().dash_apply_vec(a.ptr(X, "X", numel=P * B * B), a.ptr(g_pieces, "g_pieces", numel=P * B), P, B,
                                    a.ptr(u_pieces, "u_pieces", numel=P * B), a.stream(stream)))
