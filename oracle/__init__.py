"""CPU fp64 oracle for the batched inverse fourth root of DASH.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The GPU library and its Python binding never import it.

The arithmetic lives in ``dash_oracle.c`` (plain C, fp64, naive loops), one B x B block per call.
This wrapper only marshals numpy arrays and runs independent blocks of a stack on a thread pool
(ctypes releases the GIL during each call).  Stacking and unstacking are index permutations and
are written here directly with numpy slicing.

Citations name pages by title and section; see the header of ``dash_oracle.c`` for the tags.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dash_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile dash_oracle.c with gcc into oracle/liboracle.so (host code, no GPU)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        i, d = ctypes.c_int, ctypes.c_double
        sig = {
            "orc_matmul": (None, [i, _dp, _dp, _dp]),
            "orc_frobenius": (d, [i, _dp]),
            "orc_round_binary16": (d, [d]),
            "orc_round_bfloat16": (d, [d]),
            "orc_jacobi_eigh": (i, [i, _dp, _dp, _dp, i]),
            "orc_power_evd": (i, [i, _dp, d, _dp]),
            "orc_mpi": (d, [i, _dp, i, i, _dp, _dp]),
            "orc_mpi_half": (d, [i, _dp, i, i, _dp, _dp]),
            "orc_ndb": (None, [i, _dp, i, _dp, _dp, _dp]),
            "orc_ndb_inverse_root": (None, [i, _dp, d, i, i, _dp, _dp, _dp]),
            "orc_cn_inverse_root": (None, [i, _dp, d, i, i, _dp, _dp]),
            "orc_ndb_until": (i, [i, _dp, i, d, _dp, _dp, _dp]),
            "orc_ndb_inverse_root_until": (None, [i, _dp, d, i, i, d, _dp, _dp, _dp, _ip]),
            "orc_cn_until": (i, [i, _dp, d, i, i, d, _dp, _dp]),
            "orc_ndb_half_inverse_root": (None, [i, _dp, d, i, i, i, _dp]),
            "orc_ndb_lowp_inverse_root": (None, [i, _dp, d, i, i, i, i, _dp]),
            "orc_cheb_coeffs": (None, [i, d, d, d, _dp]),
            "orc_clenshaw": (None, [i, _dp, i, _dp, d, d, _dp]),
            "orc_cheb_inverse_root": (None, [i, _dp, d, i, d, d, _dp]),
            "orc_update_stats": (None, [i, _dp, d, _dp, _dp]),
            "orc_apply": (None, [i, _dp, _dp, _dp, _dp]),
            "orc_mpi_shifted": (d, [i, _dp, d, i, i, _dp, _dp]),
            "orc_update_stats_vec": (None, [i, _dp, d, _dp]),
            "orc_apply_vec": (None, [i, _dp, _dp, _dp]),
            "orc_ndb_inverse_sqrt": (None, [i, _dp, d, i, _dp]),
            "orc_residual_probe": (d, [i, _dp, _dp, i, _dp]),
            "orc_routed_inverse_root": (i, [i, _dp, d, i, d, d, i, i, _dp, d, i, _dp, _dp, _dp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def workers() -> int:
    """Host cores available to this process (the thread count the oracle uses)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _null():
    return ctypes.cast(None, _dp)


def _over_blocks(fn, n_blocks: int, threads: int | None = None):
    """Run fn(b) for every block b on a thread pool; results in block order."""
    threads = threads or workers()
    if n_blocks == 1 or threads == 1:
        return [fn(b) for b in range(n_blocks)]
    with ThreadPoolExecutor(max_workers=min(threads, n_blocks)) as ex:
        return list(ex.map(fn, range(n_blocks)))


def _as_stack(A):
    A = _f64(A)
    single = A.ndim == 2
    if single:
        A = A[None]
    assert A.ndim == 3 and A.shape[1] == A.shape[2], "expected (B,B) or (N,B,B)"
    return A, single


def _per_block(x, N):
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    if x.size == 1:
        x = np.repeat(x, N)
    assert x.size == N
    return x


# ---------------------------------------------------------------------------------------------
# elementary routines
# ---------------------------------------------------------------------------------------------

def matmul(X, Y) -> np.ndarray:
    X, Y = _f64(X), _f64(Y)
    n = X.shape[0]
    Z = np.empty((n, n))
    _load().orc_matmul(n, _p(X), _p(Y), _p(Z))
    return Z


def round_binary16(x) -> np.ndarray:
    """Elementwise round-to-nearest-even to IEEE binary16, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().orc_round_binary16
    return np.array([f(float(v)) for v in x.reshape(-1)]).reshape(x.shape)


def round_bfloat16(x) -> np.ndarray:
    """Elementwise round-to-nearest-even to bfloat16, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    f = _load().orc_round_bfloat16
    return np.array([f(float(v)) for v in x.reshape(-1)]).reshape(x.shape)


# storage formats of the low-precision models
_FORMATS = {None: 0, "binary16": 1, "bfloat16": 2}


def frobenius(A) -> np.ndarray:
    """Per-block Frobenius norm s_i = ||A_i||_F (c2)."""
    A, single = _as_stack(A)
    lib = _load()
    s = np.array([lib.orc_frobenius(A.shape[1], _p(A[b])) for b in range(A.shape[0])])
    return s[0] if single else s


def jacobi_eigh(A, max_sweeps: int = 50):
    """Cyclic Jacobi eigendecomposition of one symmetric block: (w, Q, sweeps); A = Q diag(w) Q^T."""
    A = _f64(A)
    n = A.shape[0]
    w = np.empty(n)
    Q = np.empty((n, n))
    sweeps = _load().orc_jacobi_eigh(n, _p(A), _p(w), _p(Q), max_sweeps)
    return w, Q, sweeps


def power_evd(A, expo: float, threads: int | None = None) -> np.ndarray:
    """Exact A^expo of each SPD block via Jacobi EVD (c1).  Raises if a block is not SPD."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    X = np.empty_like(A)
    lib = _load()

    def one(b):
        return lib.orc_power_evd(n, _p(A[b]), float(expo), _p(X[b]))

    rcs = _over_blocks(one, N, threads)
    for b, rc in enumerate(rcs):
        if rc == 1:
            raise ValueError("block %d is not positive definite" % b)
        if rc == 2:
            raise RuntimeError("Jacobi did not converge on block %d" % b)
    return X[0] if single else X


def inverse_root_evd(A, threads: int | None = None) -> np.ndarray:
    """Exact A^{-1/4} per block (c1)."""
    return power_evd(A, -0.25, threads)


# ---------------------------------------------------------------------------------------------
# scaling (c2, c3)
# ---------------------------------------------------------------------------------------------

def mpi(A, V0, steps: int, half: bool = False, threads: int | None = None):
    """Multi-Power-Iteration scale per block (c3): returns (s[N], mu[N,k]).

    V0 is the shared (B, k) start-vector pool.  half=True models the binary16 variant."""
    A, single = _as_stack(A)
    V0 = _f64(V0)
    N, n, _ = A.shape
    k = V0.shape[1]
    assert V0.shape[0] == n
    mu = np.empty((N, k))
    lib = _load()
    fn = lib.orc_mpi_half if half else lib.orc_mpi

    def one(b):
        return fn(n, _p(A[b]), k, int(steps), _p(V0), _p(mu[b]))

    s = np.array(_over_blocks(one, N, threads))
    return (s[0], mu[0]) if single else (s, mu)


# ---------------------------------------------------------------------------------------------
# solvers (c4 - c7)
# ---------------------------------------------------------------------------------------------

def ndb(M, steps: int):
    """One NDB call on a single block (c4): (Y -> M^{1/2}, Z -> M^{-1/2}, monitor[steps])."""
    M = _f64(M)
    n = M.shape[0]
    Y, Z, mon = np.empty((n, n)), np.empty((n, n)), np.empty(max(steps, 1))
    _load().orc_ndb(n, _p(M), int(steps), _p(Y), _p(Z), _p(mon))
    return Y, Z, mon[:steps]


def ndb_inverse_root(A, s, iters1: int, iters2: int, threads: int | None = None, want_sqrt: bool = False):
    """A^{-1/4} by two composed NDB calls (c5).  Returns (X, sqrt or None, monitor[N, iters1+iters2])."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    R = np.empty_like(A) if want_sqrt else None
    mon = np.empty((N, max(iters1 + iters2, 1)))
    lib = _load()

    def one(b):
        lib.orc_ndb_inverse_root(n, _p(A[b]), float(s[b]), int(iters1), int(iters2), _p(X[b]),
                                 _p(R[b]) if want_sqrt else _null(), _p(mon[b]))

    _over_blocks(one, N, threads)
    mon = mon[:, : iters1 + iters2]
    if single:
        return X[0], (R[0] if want_sqrt else None), mon[0]
    return X, R, mon


def cn_inverse_root(A, s, iters: int, half_storage: bool = False, threads: int | None = None,
                    storage: str | None = None):
    """A^{-1/4} by the Coupled-Newton p=4 iteration (c6).  Returns (X, monitor[N, iters]).
    storage: None (exact), "binary16" or "bfloat16" rounds every stored iterate to that format
    (half_storage=True is "binary16")."""
    fmt = _FORMATS[storage if storage is not None else ("binary16" if half_storage else None)]
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    mon = np.empty((N, max(iters, 1)))
    lib = _load()

    def one(b):
        lib.orc_cn_inverse_root(n, _p(A[b]), float(s[b]), int(iters), fmt, _p(X[b]), _p(mon[b]))

    _over_blocks(one, N, threads)
    mon = mon[:, :iters]
    return (X[0], mon[0]) if single else (X, mon)


def ndb_inverse_root_adaptive(A, s, max1: int, max2: int, tol: float, threads: int | None = None):
    """Composed NDB root with the per-block stopping rule (each call stops before a step k >= 1 once
    its monitor is <= tol).  Returns (X, monitor[N, max1+max2] (0 after a stop), steps[N, 2])."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    mon = np.zeros((N, max(max1 + max2, 1)))
    steps = np.zeros((N, 2), dtype=np.int32)
    lib = _load()

    def one(b):
        lib.orc_ndb_inverse_root_until(n, _p(A[b]), float(s[b]), int(max1), int(max2), float(tol), _p(X[b]),
                                       _null(), _p(mon[b]), steps[b].ctypes.data_as(_ip))

    _over_blocks(one, N, threads)
    mon = mon[:, : max1 + max2]
    return (X[0], mon[0], steps[0]) if single else (X, mon, steps)


def cn_inverse_root_adaptive(A, s, max_iters: int, tol: float, threads: int | None = None):
    """Coupled-Newton root with the per-block stopping rule.  Returns (X, monitor (0 after a stop),
    steps[N])."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    mon = np.zeros((N, max(max_iters, 1)))
    steps = np.zeros(N, dtype=np.int32)
    lib = _load()

    def one(b):
        steps[b] = lib.orc_cn_until(n, _p(A[b]), float(s[b]), int(max_iters), 0, float(tol), _p(X[b]), _p(mon[b]))

    _over_blocks(one, N, threads)
    mon = mon[:, :max_iters]
    return (X[0], mon[0], steps[0]) if single else (X, mon, steps)


def ndb_half_inverse_root(A, s, iters1: int, iters2: int, refine: int = 0, threads: int | None = None,
                          storage: str = "binary16"):
    """Composed NDB root with 2-byte iterates (storage "binary16" or "bfloat16"), then `refine`
    guarded Newton correction steps against A_s (each followed by symmetrisation).  Returns X."""
    fmt = _FORMATS[storage]
    assert fmt > 0
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    lib = _load()

    def one(b):
        lib.orc_ndb_lowp_inverse_root(n, _p(A[b]), float(s[b]), int(iters1), int(iters2), fmt, int(refine),
                                      _p(X[b]))

    _over_blocks(one, N, threads)
    return X[0] if single else X


def cheb_coeffs(degree: int, lo: float, hi: float, expo: float = -0.25) -> np.ndarray:
    """Chebyshev interpolation coefficients c_0..c_d of x^expo on [lo, hi] (c7)."""
    c = np.empty(degree + 1)
    _load().orc_cheb_coeffs(int(degree), float(lo), float(hi), float(expo), _p(c))
    return c


def clenshaw(As, c, lo: float, hi: float) -> np.ndarray:
    """sum_k c_k T_k(That) for one block by Clenshaw's recurrence (c7)."""
    As = _f64(As)
    c = _f64(c)
    n = As.shape[0]
    P = np.empty((n, n))
    _load().orc_clenshaw(n, _p(As), len(c) - 1, _p(c), float(lo), float(hi), _p(P))
    return P


def cheb_inverse_root(A, s, degree: int, lo, hi: float, threads: int | None = None) -> np.ndarray:
    """A^{-1/4} by a degree-d Chebyshev interpolant on [lo, hi] of A/s, unscaled by s^{-1/4} (c7).
    lo: one lower end for every block, or one per block."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    lo = _per_block(lo, N)
    X = np.empty_like(A)
    lib = _load()

    def one(b):
        lib.orc_cheb_inverse_root(n, _p(A[b]), float(s[b]), int(degree), float(lo[b]), float(hi), _p(X[b]))

    _over_blocks(one, N, threads)
    return X[0] if single else X


def cheb_interval_lo(s, floor: float, lam=None, theta: float = 1.0) -> np.ndarray:
    """Lower end of each block's Chebyshev interval in units of A/s: max(floor, theta lam) / s (the
    per-block reading of c7's interval)."""
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    bottom = np.full(s.shape, float(floor))
    if lam is not None:
        bottom = np.fmax(bottom, theta * np.asarray(lam, dtype=np.float64).reshape(-1))  # NaN: the floor
    return bottom / s


def mpi_shifted(A, sigma, V0, steps: int, threads: int | None = None):
    """Smallest-eigenvalue estimate per block from the power iteration on sigma I - A: returns
    (lam[N], mu[N,k]) with lam = sigma - max_j mu_j."""
    A, single = _as_stack(A)
    V0 = _f64(V0)
    N, n, _ = A.shape
    k = V0.shape[1]
    sig = _per_block(sigma, N)
    mu = np.empty((N, k))
    lib = _load()

    def one(b):
        return lib.orc_mpi_shifted(n, _p(A[b]), float(sig[b]), k, int(steps), _p(V0), _p(mu[b]))

    lam = np.array(_over_blocks(one, N, threads))
    return (lam[0], mu[0]) if single else (lam, mu)


def residual_probe(A, X, V0, threads: int | None = None) -> np.ndarray:
    """r[N]: sqrt(mean_j ||(X^4 A - I) v_j||^2) over the normalised columns v_j of V0."""
    A, single = _as_stack(A)
    X, _ = _as_stack(X)
    V0 = _f64(V0)
    N, n, _ = A.shape
    k = V0.shape[1]
    lib = _load()

    def one(b):
        return lib.orc_residual_probe(n, _p(A[b]), _p(X[b]), k, _p(V0))

    r = np.array(_over_blocks(one, N, threads))
    return r[0] if single else r


def routed_inverse_root(A, s, degree: int, floor: float, hi: float, V0, est_steps: int, tol: float, cn_iters: int,
                        threads: int | None = None):
    """Per-block solver choice: Chebyshev on [max(floor, lam/2)/s, hi] with lam the shifted power
    iteration's estimate, kept when the probe's residual is <= tol, else coupled Newton (stopping at
    tol/2).  Returns (X, route[N], lam[N], r[N]) with r the probe's residual of the Chebyshev result."""
    A, single = _as_stack(A)
    V0 = _f64(V0)
    N, n, _ = A.shape
    k = V0.shape[1]
    s = _per_block(s, N)
    X = np.empty_like(A)
    lam = np.empty(N)
    r = np.empty(N)
    lib = _load()

    def one(b):
        lp = lam[b:].ctypes.data_as(_dp)
        rp = r[b:].ctypes.data_as(_dp)
        return lib.orc_routed_inverse_root(n, _p(A[b]), float(s[b]), int(degree), float(floor), float(hi), k,
                                           int(est_steps), _p(V0), float(tol), int(cn_iters), _p(X[b]), lp, rp)

    route = np.array(_over_blocks(one, N, threads), dtype=np.int32)
    if single:
        return X[0], route[0], lam[0], r[0]
    return X, route, lam, r


# ---------------------------------------------------------------------------------------------
# surrounding steps (c8, c9, stack)
# ---------------------------------------------------------------------------------------------

def update_stats(G, beta: float, L, R, threads: int | None = None):
    """EMA statistics (c8): returns new (L, R) with L = beta L + (1-beta) G G^T, R likewise with G^T G."""
    G, single = _as_stack(G)
    L2, _ = _as_stack(L)
    R2, _ = _as_stack(R)
    L2, R2 = L2.copy(), R2.copy()
    N, n, _ = G.shape
    lib = _load()

    def one(b):
        lib.orc_update_stats(n, _p(G[b]), float(beta), _p(L2[b]), _p(R2[b]))

    _over_blocks(one, N, threads)
    return (L2[0], R2[0]) if single else (L2, R2)


def apply(XL, G, XR, threads: int | None = None) -> np.ndarray:
    """Preconditioned update U = (XL G) XR per tile (c9)."""
    G, single = _as_stack(G)
    XL, _ = _as_stack(XL)
    XR, _ = _as_stack(XR)
    N, n, _ = G.shape
    U = np.empty_like(G)
    lib = _load()

    def one(b):
        lib.orc_apply(n, _p(XL[b]), _p(G[b]), _p(XR[b]), _p(U[b]))

    _over_blocks(one, N, threads)
    return U[0] if single else U


def stack(grads, B: int) -> np.ndarray:
    """Blockify weight gradients into a (N_G, B, B) stack: weight-major, then tile row, then tile column.

    [PT] Metodologia, item 1 (gradient blocks G_ij are stacked into an (N, B, B) tensor).  The pages
    tile weights into blocks of about 1k and say nothing of edges; here a weight whose sides are not
    multiples of B gets ceil(rows/B) x ceil(cols/B) tiles and the part of an edge tile that lies
    outside the weight is zero."""
    tiles = []
    for W in grads:
        W = np.asarray(W)
        rows, cols = W.shape
        if rows < 1 or cols < 1:
            raise ValueError("empty weight %s" % (W.shape,))
        for tr in range(-(-rows // B)):
            for tc in range(-(-cols // B)):
                part = W[tr * B:(tr + 1) * B, tc * B:(tc + 1) * B]
                tile = np.zeros((B, B), dtype=W.dtype)
                tile[:part.shape[0], :part.shape[1]] = part
                tiles.append(tile)
    return np.stack(tiles)


def unstack(U, shapes, B: int):
    """Inverse of :func:`stack`: scatter (N_G, B, B) tiles back into weights of the given shapes
    (the padding of edge tiles is dropped)."""
    U = np.asarray(U)
    out, t = [], 0
    for rows, cols in shapes:
        W = np.empty((rows, cols), dtype=U.dtype)
        for tr in range(-(-rows // B)):
            for tc in range(-(-cols // B)):
                h, w = min(B, rows - tr * B), min(B, cols - tc * B)
                W[tr * B:tr * B + h, tc * B:tc * B + w] = U[t][:h, :w]
                t += 1
        out.append(W)
    assert t == U.shape[0]
    return out


# ---------------------------------------------------------------------------------------------
# 1-D parameters: pieces of B, L_p <- beta L_p + (1 - beta) g_p g_p^T, update L_p^{-1/2} g_p
# ---------------------------------------------------------------------------------------------

def stack_vec(vectors, B: int) -> np.ndarray:
    """[P, B] pieces of the vectors, vector-major, the last piece of each zero-padded."""
    out = []
    for v in vectors:
        v = _f64(v).reshape(-1)
        n = -(-v.size // B)
        pad = np.zeros(n * B)
        pad[: v.size] = v
        out.append(pad.reshape(n, B))
    return np.concatenate(out)


def unstack_vec(pieces, lens, B: int):
    """The vectors of the given lengths back from their pieces."""
    flat = _f64(pieces).reshape(-1)
    out, off = [], 0
    for n in lens:
        out.append(flat[off:off + n].copy())
        off += -(-n // B) * B
    return out


def update_stats_vec(g, beta: float, L, threads: int | None = None) -> np.ndarray:
    """L_p <- beta L_p + (1 - beta) g_p g_p^T for every piece (returns the new stack)."""
    g = _f64(g)
    L = _f64(L).copy()
    P, n = g.shape
    lib = _load()

    def one(p):
        lib.orc_update_stats_vec(n, _p(g[p]), float(beta), _p(L[p]))

    _over_blocks(one, P, threads)
    return L


def apply_vec(X, g, threads: int | None = None) -> np.ndarray:
    """u_p = X_p g_p."""
    X = _f64(X)
    g = _f64(g)
    P, n = g.shape
    u = np.empty((P, n))
    lib = _load()

    def one(p):
        lib.orc_apply_vec(n, _p(X[p]), _p(g[p]), _p(u[p]))

    _over_blocks(one, P, threads)
    return u


def ndb_inverse_sqrt(A, s, iters: int, threads: int | None = None) -> np.ndarray:
    """A^{-1/2} by one NDB call on A/s (its Z), unscaled by s^{-1/2}."""
    A, single = _as_stack(A)
    N, n, _ = A.shape
    s = _per_block(s, N)
    X = np.empty_like(A)
    lib = _load()

    def one(b):
        lib.orc_ndb_inverse_sqrt(n, _p(A[b]), float(s[b]), int(iters), _p(X[b]))

    _over_blocks(one, N, threads)
    return X[0] if single else X
