"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random matrices and builds the
symmetric positive-definite test stacks described below.  Both the GPU path and the CPU oracle
receive the SAME fp32 values from here (the oracle widens them to fp64).

Workloads (shapes of the pages' Llama setup: embedding 2048, block size about 1024, preconditioner
blocks of L and R stacked in one tensor -- DASH technical summary (gist.science, pt), "Resultados
Experimentais" and "Metodologia"; quant_prune_distill post 646, body):

* tiny stack        N=4,  B=64:   A_i = G_i G_i^T / 128 + 1e-4 I, G_i (64 x 128) iid N(0,1).
* conditioned stack N=16, B=256:  A_i = Q_i diag(lam_i) Q_i^T, Q_i from QR of a Gaussian matrix,
                                  lam log-uniform on [1e-4, 1] with its min set to 1e-4 and max to 1.
* gram stack        N=3072, B=1024: A = G G^T / 1024 + 1e-6 I, G iid N(0, 1e-3^2) (built on the GPU by torch).
* llama gradients   24 layers x (4 x 2048x2048 + 3 x 2048x8192) tiles into 1536 blocks of 1024 x 1024.
"""
from __future__ import annotations

import numpy as np

SEED_TINY = 1
SEED_CONDITIONED = 2
SEED_GRAM = 3
SEED_GRADS = 5
SEED_START = 7


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tiny_stack(seed: int = SEED_TINY, N: int = 4, B: int = 64, cols: int = 128, eps: float = 1e-4) -> np.ndarray:
    """(N, B, B) fp32 stack A_i = G_i G_i^T / cols + eps I, built in fp64 and rounded once."""
    g = rng(seed)
    out = np.empty((N, B, B), dtype=np.float32)
    for i in range(N):
        G = g.standard_normal((B, cols))
        A = G @ G.T / cols + eps * np.eye(B)
        A = 0.5 * (A + A.T)
        out[i] = A.astype(np.float32)
    return out


def haar_orthogonal(g: np.random.Generator, B: int) -> np.ndarray:
    """Q factor of a Gaussian B x B matrix with the sign fix diag(R) > 0."""
    Q, R = np.linalg.qr(g.standard_normal((B, B)))
    return Q * np.sign(np.diag(R))[None, :]


def conditioned_stack(seed: int = SEED_CONDITIONED, N: int = 16, B: int = 256, lam_min: float = 1e-4,
                      lam_max: float = 1.0):
    """(A fp32 (N,B,B), Q fp64 (N,B,B), lam fp64 (N,B)) with A_i = Q_i diag(lam_i) Q_i^T."""
    g = rng(seed)
    A = np.empty((N, B, B), dtype=np.float32)
    Qs = np.empty((N, B, B))
    lams = np.empty((N, B))
    for i in range(N):
        Q = haar_orthogonal(g, B)
        lam = np.exp(g.uniform(np.log(lam_min), np.log(lam_max), B))
        lam[np.argmin(lam)] = lam_min
        lam[np.argmax(lam)] = lam_max
        M = (Q * lam[None, :]) @ Q.T
        A[i] = (0.5 * (M + M.T)).astype(np.float32)
        Qs[i], lams[i] = Q, lam
    return A, Qs, lams


def known_spectrum_stack(seed: int, N: int, B: int, lam_min: float, lam_max: float):
    """Like conditioned_stack but returns the fp64 matrices too: (A64, Q, lam)."""
    g = rng(seed)
    A = np.empty((N, B, B))
    Qs = np.empty((N, B, B))
    lams = np.empty((N, B))
    for i in range(N):
        Q = haar_orthogonal(g, B)
        lam = np.exp(g.uniform(np.log(lam_min), np.log(lam_max), B))
        lam[np.argmin(lam)] = lam_min
        lam[np.argmax(lam)] = lam_max
        M = (Q * lam[None, :]) @ Q.T
        A[i] = 0.5 * (M + M.T)
        Qs[i], lams[i] = Q, lam
    return A, Qs, lams


def start_vectors(B: int, k: int = 32, seed: int = SEED_START) -> np.ndarray:
    """Shared (B, k) pool of power-iteration start vectors, iid N(0,1), fp32."""
    return rng(seed).standard_normal((B, k)).astype(np.float32)


def start_pool_counter(B: int, k: int, seed: int) -> np.ndarray:
    """The (B, k) start pool drawn from a counter-based SplitMix64 stream (Steele, Lea and Flood, 2014):
    output n of the stream started at `seed` is mix(seed + n * 0x9E3779B97F4A7C15); element e = i k + j
    takes the top 22 bits u_q of outputs 3e + q (q = 1, 2, 3) and is (u_1 + u_2 + u_3 - 1.5 * 2^22) * 2^-22,
    exact in fp32.  The GPU library draws the same pool when dash_scale is given no start vectors."""
    e = np.arange(B * k, dtype=np.uint64)
    total = np.zeros(B * k, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for q in (1, 2, 3):
            z = np.uint64(seed) + (np.uint64(3) * e + np.uint64(q)) * np.uint64(0x9E3779B97F4A7C15)
            z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
            z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
            z = z ^ (z >> np.uint64(31))
            total += z >> np.uint64(42)
    v = (total.astype(np.float32) - np.float32(6291456.0)) * np.float32(2.0 ** -22)
    return v.reshape(B, k)


def gaussian(shape, seed: int, std: float = 1.0) -> np.ndarray:
    return (std * rng(seed).standard_normal(shape)).astype(np.float32)


def llama_weight_shapes(layers: int = 24, d: int = 2048, ffn: int = 8192):
    """Per layer: four d x d attention weights and three d x ffn MLP weights (row-major)."""
    shapes = []
    for _ in range(layers):
        shapes += [(d, d)] * 4 + [(d, ffn)] * 3
    return shapes


def num_tiles(shapes, B: int) -> int:
    """Tiles of a stack of weights of these shapes (edge tiles of non-multiple sides included)."""
    return sum((-(-r // B)) * (-(-c // B)) for r, c in shapes)


# ---------------------------------------------------------------------------------------------------
# large stacks, built on the GPU with torch (harness only; torch is plumbing for memory here)
# ---------------------------------------------------------------------------------------------------

def gram_stack_torch(N: int, B: int, seed: int = SEED_GRAM, device="cuda", std: float = 1e-3,
                     eps: float = 1e-6, chunk: int = 64):
    """(N, B, B) fp32 torch stack A = G G^T / B + eps I, G iid N(0, std^2), exactly symmetric."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    A = torch.empty((N, B, B), dtype=torch.float32, device=device)
    eye = torch.eye(B, dtype=torch.float32, device=device)
    for i0 in range(0, N, chunk):
        n = min(chunk, N - i0)
        G = torch.randn((n, B, B), generator=gen, device=device, dtype=torch.float32) * std
        M = torch.matmul(G, G.transpose(1, 2).contiguous()) / B
        M = 0.5 * (M + M.transpose(1, 2))
        A[i0:i0 + n] = M + eps * eye
        del G, M
    return A


def gaussian_torch(shape, seed: int, device="cuda", std: float = 1.0):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std
