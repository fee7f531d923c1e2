"""Write tests/golden/closed_forms.json: small examples whose answers follow from the mathematics alone.

The pages about DASH print no worked example, so every fixture here is a textbook closed form,
derived in exact rational arithmetic (``fractions``).  Nothing here calls the oracle or the GPU
library.  Run:  python tests/golden/make_closed_forms.py

Fixtures
--------
* inverse fourth roots A^{-1/4} (and square roots A^{1/2}) of SPD matrices built as
  H diag(lam) H^T with H orthogonal and lam powers of 16, so that lam^{-1/4} and lam^{1/2} are exact;
* Rayleigh quotients of the power iteration on diagonal matrices: after T products from start
  vector v, mu = sum_i lam_i^{2T-1} v_i^2 / sum_i lam_i^{2T-2} v_i^2 (normalisation does not change it);
* Chebyshev coefficients of x^2 on [lo, hi]: with x = a t + b, a = (hi-lo)/2, b = (hi+lo)/2,
  x^2 = (b^2 + a^2/2) T_0 + 2ab T_1 + (a^2/2) T_2, exactly.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))


def mat_from_eig(H, lam):
    """sum_k lam_k h_k h_k^T / ||h_k||^2 for orthogonal (unnormalised) columns h_k (rows of H here)."""
    n = len(lam)
    out = [[F(0)] * n for _ in range(n)]
    for h, l in zip(H, lam):
        nrm = sum(F(x) * x for x in h)
        for i in range(n):
            for j in range(n):
                out[i][j] += l * F(h[i]) * h[j] / nrm
    return out


def fourth_root_inv(l: F) -> F:
    # l is a power of 16 (possibly negative exponent): l^{-1/4} is a power of 2
    for e in range(-12, 13):
        if F(16) ** e == l:
            return F(2) ** (-e)
    raise ValueError(l)


def sqrt_exact(l: F) -> F:
    for e in range(-12, 13):
        if F(16) ** e == l:
            return F(4) ** e
    raise ValueError(l)


def as_float(M):
    return [[float(x) for x in row] for row in M]


def spd_fixture(name, H, lam, note):
    lam = [F(x) for x in lam]
    A = mat_from_eig(H, lam)
    X = mat_from_eig(H, [fourth_root_inv(l) for l in lam])
    R = mat_from_eig(H, [sqrt_exact(l) for l in lam])
    return {"name": name, "A": as_float(A), "inv_fourth_root": as_float(X), "sqrt": as_float(R),
            "lambda_max": float(max(lam)), "note": note}


def main():
    roots = []
    e = [[1 if i == j else 0 for j in range(4)] for i in range(4)]
    roots.append(spd_fixture("diag4", e, [16, 1, 256, F(1, 16)],
                             "diagonal: A^{-1/4} = diag(lam^{-1/4})"))
    roots.append(spd_fixture("rot2", [[1, 1], [1, -1]], [16, 1],
                             "eigenvectors (1,1)/sqrt2 and (1,-1)/sqrt2; A = [[8.5,7.5],[7.5,8.5]]"))
    hadamard = [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]
    roots.append(spd_fixture("hadamard4", hadamard, [256, 16, 1, F(1, 16)],
                             "H diag(256,16,1,1/16) H^T / 4 with the 4x4 Hadamard matrix H"))
    sylv = [[1]]
    for _ in range(3):  # Sylvester construction of the 8x8 Hadamard matrix
        sylv = [r + r for r in sylv] + [r + [-x for x in r] for r in sylv]
    roots.append(spd_fixture("hadamard8", sylv, [1, F(1, 16), 16, F(1, 256), 1, 16, F(1, 16), 256],
                             "8x8 Sylvester-Hadamard eigenvectors, spectrum 1/256 .. 256 (kappa 65536)"))

    mpi = []

    def mu_closed(lam, v, T):
        lam = [F(x) for x in lam]
        v = [F(x) for x in v]
        num = sum(l ** (2 * T - 1) * x * x for l, x in zip(lam, v))
        den = sum(l ** (2 * T - 2) * x * x for l, x in zip(lam, v))
        return num / den

    for lam, V, T in [([4, 2, 1], [[1, 1], [1, 0], [1, 1]], 2),
                      ([4, 2, 1], [[1, 1], [1, 0], [1, 1]], 1),
                      ([3, F(1, 2), 5, 1], [[1, 0, 2], [2, 1, 0], [1, 0, 1], [-1, 3, 1]], 4)]:
        cols = [[row[j] for row in V] for j in range(len(V[0]))]
        mus = [mu_closed(lam, c, T) for c in cols]
        mpi.append({"lam": [float(F(x)) for x in lam], "V0": [[float(F(x)) for x in r] for r in V], "T": T,
                    "mu": [float(m) for m in mus], "mu_fraction": [str(m) for m in mus],
                    "s": float(max(mus))})

    cheb = []
    for lo, hi in [(F(0), F(2)), (F(1, 4), F(5, 4)), (F(-3), F(5))]:
        a, b = (hi - lo) / 2, (hi + lo) / 2
        c = [b * b + a * a / 2, 2 * a * b, a * a / 2]
        cheb.append({"f": "x^2", "lo": float(lo), "hi": float(hi), "coeffs": [float(x) for x in c]})

    out = {
        "source": "closed forms from the mathematics (the pages print no worked example); "
                  "written by tests/golden/make_closed_forms.py with exact rational arithmetic",
        "inverse_roots": roots,
        "power_iteration": mpi,
        "chebyshev": cheb,
    }
    with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
