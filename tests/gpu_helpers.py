"""Shared helpers of the GPU parity tests (host-side arithmetic is fp64 numpy, never the GPU path)."""
import numpy as np
import torch

import matrix_inverse_roots_amd as dash
import oracle

DEV = torch.device("cuda:0")

# gates (fp32: residual 1e-3 and iterate parity 1e-4; fp16 operands: residual 5e-3)
R_FP32 = 1e-3
R_FP16 = 5e-3
ITERATE_TOL = 1e-4


def to_dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def to_host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def rel_err(X, R):
    """per-block ||X - R||_F / ||R||_F"""
    X, R = np.asarray(X, np.float64), np.asarray(R, np.float64)
    if X.ndim == 2:
        X, R = X[None], R[None]
    return np.linalg.norm(X - R, axis=(1, 2)) / np.linalg.norm(R, axis=(1, 2))


def residual(X, A):
    """per-block ||X^4 A - I||_F / sqrt(B), in fp64 on the host"""
    X, A = np.asarray(X, np.float64), np.asarray(A, np.float64)
    if X.ndim == 2:
        X, A = X[None], A[None]
    B = A.shape[-1]
    X2 = X @ X
    return np.linalg.norm(X2 @ X2 @ A - np.eye(B), axis=(1, 2)) / np.sqrt(B)


def power_scale(A, V0, steps=10, prec=dash.DASH_FP32):
    N, B = A.shape[0], A.shape[1]
    s = torch.empty(N, device=DEV)
    ws = dash.workspace(dash.DASH_OP_SCALE, N, B, prec, V0.shape[1], device=DEV)
    dash.dash_scale(A, N, B, dash.DASH_SCALE_POWER, prec, V0.shape[1], steps, V0, s, ws)
    return s


def host_power_scale(A, V0, steps=10):
    """The oracle's power-iteration scale per block rounded to fp32, on the device: the scale that a
    solver test feeds to both its GPU solve and the oracle (no oracle input comes from the HIP path)."""
    s, _ = oracle.mpi(np.asarray(A, np.float64), np.asarray(V0, np.float64), steps)
    return to_dev(np.asarray(s, np.float32).reshape(-1))


def host_frob_scale(A):
    """The oracle's Frobenius scale per block rounded to fp32, on the device."""
    return to_dev(np.asarray(oracle.frobenius(np.asarray(A, np.float64)), np.float32).reshape(-1))


def frob_scale(A):
    N, B = A.shape[0], A.shape[1]
    s = torch.empty(N, device=DEV)
    dash.dash_scale(A, N, B, dash.DASH_SCALE_FROBENIUS, dash.DASH_FP32, 0, 0, None, s, None)
    return s


def ndb(A, s, it1, it2, want_sqrt=False, want_monitor=False):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    R = torch.empty_like(A) if want_sqrt else None
    mon = torch.empty((N, it1 + it2), device=DEV) if want_monitor else None
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, device=DEV)
    dash.dash_inverse_root_ndb(A, s, N, B, it1, it2, X, sqrt_out=R, monitor=mon, status=status, ws=ws)
    return X, R, mon, status


def cn(A, s, iters, prec=dash.DASH_FP32, want_monitor=False):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    mon = torch.empty((N, iters), device=DEV) if want_monitor else None
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CN, N, B, prec, device=DEV)
    dash.dash_inverse_root_cn(A, s, N, B, 4, iters, prec, X, monitor=mon, status=status, ws=ws)
    return X, mon, status


def cheb(A, s, degree, lo, hi):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CHEB, N, B, device=DEV)
    dash.dash_inverse_root_cheb(A, s, N, B, degree, lo, hi, X, status=status, ws=ws)
    return X, status


def evd(A, max_sweeps=20, refine=0, prec=None):
    """(X, eigenvalues, sweeps, status) of the block-Jacobi eigendecomposition solver (prec None:
    the fp32 entry point; else the entry point that takes the first pass's precision)."""
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    w = torch.empty((N, B), device=DEV)
    sweeps = torch.empty(N, dtype=torch.int32, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_EVD, N, B, device=DEV)
    if prec is None:
        dash.dash_inverse_root_evd(A, N, B, max_sweeps, refine, X, eigvals=w, sweeps=sweeps, status=status, ws=ws)
    else:
        dash.dash_inverse_root_evd_prec(A, N, B, max_sweeps, refine, prec, X, eigvals=w, sweeps=sweeps,
                                        status=status, ws=ws)
    return X, w, sweeps, status


def ndb_adaptive(A, s, max1, max2, tol):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    mon = torch.empty((N, max1 + max2), device=DEV)
    steps = torch.empty((N, 2), dtype=torch.int32, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_NDB, N, B, device=DEV)
    dash.dash_inverse_root_ndb_adaptive(A, s, N, B, max1, max2, tol, X, mon, steps=steps, status=status, ws=ws)
    return X, mon, steps, status


def cn_adaptive(A, s, max_iters, tol, prec=dash.DASH_FP32):
    N, B = A.shape[0], A.shape[1]
    X = torch.empty_like(A)
    mon = torch.empty((N, max_iters), device=DEV)
    steps = torch.empty(N, dtype=torch.int32, device=DEV)
    status = torch.empty(N, dtype=torch.int32, device=DEV)
    ws = dash.workspace(dash.DASH_OP_CN, N, B, prec, device=DEV)
    dash.dash_inverse_root_cn_adaptive(A, s, N, B, 4, max_iters, tol, prec, X, mon, steps=steps, status=status,
                                       ws=ws)
    return X, mon, steps, status
