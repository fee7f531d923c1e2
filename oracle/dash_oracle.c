/*
 * dash_oracle.c -- plain, slow CPU oracle (fp64) for the batched inverse fourth root of DASH.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The GPU library never links, includes or calls it,
 * and it shares no code with the GPU library.
 *
 * Every routine works on ONE B x B block held row-major in fp64.  Products are naive i-k-j loops,
 * no BLAS, no blocking, no SIMD intrinsics, so that each step can be checked against the pages by eye.
 * Batching over the stack is done by the Python wrapper (one block per thread).
 *
 * Pages cited (by title and section):
 *   [PT] "Resumo Técnico: DASH – Shampoo Mais Rápido via Pré-condicionamento de Blocos em Lote e
 *        Solvers de Raiz Inversa Eficientes" (gist.science/pt/paper/2602.02016)
 *   [FR] French summary of the same paper (gist.science/fr/paper/2602.02016), "Méthodologie"
 *   [TG] quant_prune_distill post 646 (tgviewer.app), commentary on DASH
 *   [AB] arxivdaily.com/papers/2602.02016, English abstract
 *
 * The pages give no formulas.  Where a step is left open the reading taken here is stated at the
 * routine; each such reading is listed again in the design notes of the repository.
 *
 * Parity pins: every routine below is pinned by tests that do not re-run this code (closed forms,
 * scalar recurrences on known spectra, brute force on 4x4 blocks, library routines on special
 * cases).  No routine is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IDX(i, j, n) ((size_t)(i) * (size_t)(n) + (size_t)(j))

/* ------------------------------------------------------------------------------------------------
 * Basic matrix helpers
 * ---------------------------------------------------------------------------------------------- */

/* Z = X * Y for n x n row-major matrices; naive i-k-j loop.  Z must not alias X or Y. */
void orc_matmul(int n, const double* X, const double* Y, double* Z) {
  for (size_t e = 0; e < (size_t)n * n; ++e) Z[e] = 0.0;
  for (int i = 0; i < n; ++i)
    for (int k = 0; k < n; ++k) {
      const double xik = X[IDX(i, k, n)];
      for (int j = 0; j < n; ++j) Z[IDX(i, j, n)] += xik * Y[IDX(k, j, n)];
    }
}

static void set_identity(int n, double* X, double c) {
  for (size_t e = 0; e < (size_t)n * n; ++e) X[e] = 0.0;
  for (int i = 0; i < n; ++i) X[IDX(i, i, n)] = c;
}

static double dist_to_identity(int n, const double* P) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      const double d = P[IDX(i, j, n)] - (i == j ? 1.0 : 0.0);
      acc += d * d;
    }
  return sqrt(acc) / sqrt((double)n);
}

/* Frobenius norm ||A||_F = sqrt(sum_ij A_ij^2).
 * [PT] Definição do Problema, item 3 (Frobenius scaling is the current default); [TG] body
 * (Frobenius norm can be noticeably larger than the spectral norm). */
double orc_frobenius(int n, const double* A) {
  double acc = 0.0;
  for (size_t e = 0; e < (size_t)n * n; ++e) acc += A[e] * A[e];
  return sqrt(acc);
}

/* Round x to the nearest IEEE 754 binary16 value (ties to even) and return it as a double.
 * Written from the binary16 format definition: 11 significant bits, normal exponents -14..15,
 * subnormal quantum 2^-24, largest finite 65504. */
double orc_round_binary16(double x) {
  if (isnan(x)) return x;
  const double ax = fabs(x);
  if (ax >= 65520.0) return copysign(INFINITY, x); /* halfway to 2^16 and above round to inf */
  if (ax == 0.0) return x;
  int ex;
  frexp(ax, &ex);                   /* ax = m * 2^ex, m in [0.5, 1) => floor(log2 ax) = ex - 1 */
  int e = ex - 1;
  if (e < -14) e = -14;             /* subnormal range shares the quantum of the smallest binade */
  const double quantum = ldexp(1.0, e - 10);
  const double r = nearbyint(ax / quantum) * quantum; /* default mode: ties to even */
  return copysign(r, x);
}

/* Round x to the nearest bfloat16 value (ties to even) and return it as a double.  Written from
 * the bfloat16 format definition: 8 significant bits and the exponent range of binary32 (normal
 * exponents -126..127, subnormal quantum 2^-133, largest finite (2 - 2^-7) 2^127). */
double orc_round_bfloat16(double x) {
  if (isnan(x)) return x;
  const double ax = fabs(x);
  if (ax >= ldexp(2.0 - ldexp(1.0, -8), 127)) return copysign(INFINITY, x); /* halfway to 2^128 and above */
  if (ax == 0.0) return x;
  int ex;
  frexp(ax, &ex);
  int e = ex - 1;
  if (e < -126) e = -126;
  const double quantum = ldexp(1.0, e - 7);
  const double r = nearbyint(ax / quantum) * quantum; /* default mode: ties to even */
  return copysign(r, x);
}

/* storage formats of the low-precision models: 0 exact, 1 binary16, 2 bfloat16 */
static double round_fmt(int fmt, double x) {
  return fmt == 1 ? orc_round_binary16(x) : (fmt == 2 ? orc_round_bfloat16(x) : x);
}

/* ------------------------------------------------------------------------------------------------
 * c1: exact root by cyclic Jacobi eigendecomposition.
 * The eigendecomposition is the default root solver of Distributed Shampoo ([PT] Definição do
 * Problema, item 2; [TG] body).  Here it only provides the exact reference A^{p}.
 * ---------------------------------------------------------------------------------------------- */

/* Eigen-decompose symmetric A = Q diag(w) Q^T.  Cyclic Jacobi: pivots (p,q) row by row; each
 * rotation zeroes A_pq.  Stops when off(A) <= 1e-15 ||A||_F or after max_sweeps sweeps.
 * Q is row-major with eigenvectors in its COLUMNS.  Returns the number of sweeps used, or -1 if
 * the tolerance was not met. */
int orc_jacobi_eigh(int n, const double* A_in, double* w, double* Q, int max_sweeps) {
  double* A = (double*)malloc(sizeof(double) * (size_t)n * n);
  memcpy(A, A_in, sizeof(double) * (size_t)n * n);
  set_identity(n, Q, 1.0);
  const double fro = orc_frobenius(n, A);
  int sweep = 0, ok = 0;
  for (;;) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = 0; q < n; ++q)
        if (p != q) off += A[IDX(p, q, n)] * A[IDX(p, q, n)];
    if (sqrt(off) <= 1e-15 * fro) { ok = 1; break; }
    if (sweep == max_sweeps) break;
    ++sweep;
    for (int p = 0; p < n - 1; ++p)
      for (int q = p + 1; q < n; ++q) {
        const double apq = A[IDX(p, q, n)];
        if (apq == 0.0) continue;
        /* rotation J = I except J_pp = J_qq = c, J_pq = s, J_qp = -s, chosen so (J^T A J)_pq = 0 */
        const double theta = (A[IDX(q, q, n)] - A[IDX(p, p, n)]) / (2.0 * apq);
        double t;
        if (fabs(theta) > 1e150) t = 0.5 / theta; /* theta^2 would overflow; t ~ 1/(2 theta) */
        else t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0);
        const double s = t * c;
        /* A <- A J (columns p, q) */
        for (int r = 0; r < n; ++r) {
          const double arp = A[IDX(r, p, n)], arq = A[IDX(r, q, n)];
          A[IDX(r, p, n)] = c * arp - s * arq;
          A[IDX(r, q, n)] = s * arp + c * arq;
        }
        /* A <- J^T A (rows p, q) */
        for (int r = 0; r < n; ++r) {
          const double apr = A[IDX(p, r, n)], aqr = A[IDX(q, r, n)];
          A[IDX(p, r, n)] = c * apr - s * aqr;
          A[IDX(q, r, n)] = s * apr + c * aqr;
        }
        A[IDX(p, q, n)] = 0.0;
        A[IDX(q, p, n)] = 0.0;
        /* Q <- Q J */
        for (int r = 0; r < n; ++r) {
          const double qrp = Q[IDX(r, p, n)], qrq = Q[IDX(r, q, n)];
          Q[IDX(r, p, n)] = c * qrp - s * qrq;
          Q[IDX(r, q, n)] = s * qrp + c * qrq;
        }
      }
  }
  for (int i = 0; i < n; ++i) w[i] = A[IDX(i, i, n)];
  free(A);
  return ok ? sweep : -1;
}

/* X = Q diag(w_i^expo) Q^T from an eigendecomposition of A (expo = -1/4 gives the inverse fourth
 * root).  Returns 0 on success, 1 if some eigenvalue is <= 0 (A not SPD: no real root), 2 if the
 * Jacobi sweep limit was hit. */
int orc_power_evd(int n, const double* A, double expo, double* X) {
  double* w = (double*)malloc(sizeof(double) * n);
  double* Q = (double*)malloc(sizeof(double) * (size_t)n * n);
  int rc = 0;
  if (orc_jacobi_eigh(n, A, w, Q, 50) < 0) rc = 2;
  for (int i = 0; i < n && rc == 0; ++i)
    if (!(w[i] > 0.0)) rc = 1;
  if (rc == 0) {
    for (int i = 0; i < n; ++i) w[i] = pow(w[i], expo);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int k = 0; k < n; ++k) acc += Q[IDX(i, k, n)] * w[k] * Q[IDX(j, k, n)];
        X[IDX(i, j, n)] = acc;
      }
  }
  free(w);
  free(Q);
  return rc;
}

/* ------------------------------------------------------------------------------------------------
 * c3: Multi-Power-Iteration scaling.
 * [PT] Metodologia, item 2, "Multi-Power-Iteration" bullet (up to 32 start vectors run in parallel
 * estimate lambda_max); [TG] body (spectral-norm estimate from the Rayleigh quotient).
 * Readings: every column is normalised at every step; the Rayleigh quotient v^T A v / v^T v comes
 * from the last product; s = max over columns; no safety factor.
 * V0 is B x k row-major (column j is start vector j); mu receives the k Rayleigh quotients.
 * ---------------------------------------------------------------------------------------------- */
double orc_mpi(int n, const double* A, int k, int T, const double* V0, double* mu) {
  double* V = (double*)malloc(sizeof(double) * (size_t)n * k);
  double* W = (double*)malloc(sizeof(double) * (size_t)n * k);
  for (int j = 0; j < k; ++j) {
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) nrm += V0[IDX(i, j, k)] * V0[IDX(i, j, k)];
    nrm = sqrt(nrm);
    for (int i = 0; i < n; ++i) V[IDX(i, j, k)] = V0[IDX(i, j, k)] / nrm;
  }
  for (int t = 1; t <= T; ++t) {
    /* W = A V */
    for (size_t e = 0; e < (size_t)n * k; ++e) W[e] = 0.0;
    for (int i = 0; i < n; ++i)
      for (int l = 0; l < n; ++l) {
        const double ail = A[IDX(i, l, n)];
        for (int j = 0; j < k; ++j) W[IDX(i, j, k)] += ail * V[IDX(l, j, k)];
      }
    for (int j = 0; j < k; ++j) {
      double vw = 0.0, vv = 0.0, ww = 0.0;
      for (int i = 0; i < n; ++i) {
        vw += V[IDX(i, j, k)] * W[IDX(i, j, k)];
        vv += V[IDX(i, j, k)] * V[IDX(i, j, k)];
        ww += W[IDX(i, j, k)] * W[IDX(i, j, k)];
      }
      mu[j] = vw / vv; /* Rayleigh quotient v^T A v / v^T v */
      if (t < T) {
        const double nw = sqrt(ww);
        for (int i = 0; i < n; ++i) V[IDX(i, j, k)] = W[IDX(i, j, k)] / nw;
      }
    }
  }
  double s = mu[0];
  for (int j = 1; j < k; ++j)
    if (mu[j] > s) s = mu[j];
  free(V);
  free(W);
  return s;
}

/* Half-precision Multi-Power-Iteration ([PT] Principais Contribuições, item 4: an efficient
 * half-precision power iteration).  Reading: e = ceil(log2 max_i A_ii); the operand is
 * A_h = binary16(A * 2^-e) (round to nearest even); the iterate V is stored in binary16 after each
 * normalisation; products, norms and Rayleigh quotients are exact here (fp64); s = 2^e max_j mu_j.
 * Returns 0 for a block whose diagonal maximum is not positive. */
double orc_mpi_half(int n, const double* A, int k, int T, const double* V0, double* mu) {
  double dmax = A[0];
  for (int i = 1; i < n; ++i)
    if (A[IDX(i, i, n)] > dmax) dmax = A[IDX(i, i, n)];
  if (!(dmax > 0.0)) {
    for (int j = 0; j < k; ++j) mu[j] = 0.0;
    return 0.0;
  }
  const int e = (int)ceil(log2(dmax));
  double* Ah = (double*)malloc(sizeof(double) * (size_t)n * n);
  double* V = (double*)malloc(sizeof(double) * (size_t)n * k);
  double* W = (double*)malloc(sizeof(double) * (size_t)n * k);
  for (size_t q = 0; q < (size_t)n * n; ++q) Ah[q] = orc_round_binary16(ldexp(A[q], -e));
  for (int j = 0; j < k; ++j) {
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) nrm += V0[IDX(i, j, k)] * V0[IDX(i, j, k)];
    nrm = sqrt(nrm);
    for (int i = 0; i < n; ++i) V[IDX(i, j, k)] = orc_round_binary16(V0[IDX(i, j, k)] / nrm);
  }
  for (int t = 1; t <= T; ++t) {
    for (size_t q = 0; q < (size_t)n * k; ++q) W[q] = 0.0;
    for (int i = 0; i < n; ++i)
      for (int l = 0; l < n; ++l) {
        const double ail = Ah[IDX(i, l, n)];
        for (int j = 0; j < k; ++j) W[IDX(i, j, k)] += ail * V[IDX(l, j, k)];
      }
    for (int j = 0; j < k; ++j) {
      double vw = 0.0, vv = 0.0, ww = 0.0;
      for (int i = 0; i < n; ++i) {
        vw += V[IDX(i, j, k)] * W[IDX(i, j, k)];
        vv += V[IDX(i, j, k)] * V[IDX(i, j, k)];
        ww += W[IDX(i, j, k)] * W[IDX(i, j, k)];
      }
      mu[j] = ldexp(vw / vv, e); /* the stored v is unit-norm only up to binary16 rounding */
      if (t < T) {
        const double nw = sqrt(ww);
        for (int i = 0; i < n; ++i) V[IDX(i, j, k)] = orc_round_binary16(W[IDX(i, j, k)] / nw);
      }
    }
  }
  double s = mu[0];
  for (int j = 1; j < k; ++j)
    if (mu[j] > s) s = mu[j];
  free(Ah);
  free(V);
  free(W);
  return s;
}

/* ------------------------------------------------------------------------------------------------
 * c4: one Newton-Denman-Beavers call.
 * [PT] Metodologia, item 2, "Iteração de Newton-Denman-Beavers": one iteration yields both the
 * square root and the inverse square root, at three matrix products per step.
 * Reading: the coupled, inverse-free Newton-Schulz form of the Denman-Beavers iteration
 * (Higham, Functions of Matrices, 2008, ch. 6), with this operand order:
 *     Y_0 = M, Z_0 = I;   P = Z_k Y_k,  S = (3 I - P) / 2,  Y_{k+1} = Y_k S,  Z_{k+1} = S Z_k.
 * Y_T -> M^{1/2}, Z_T -> M^{-1/2}.  The pages' first-step saving (P = M because Z_0 = I) changes
 * no value, so this plain form runs every step in full.
 * monitor[k] (optional) = ||P_k - I||_F / sqrt(n).
 * ---------------------------------------------------------------------------------------------- */
/* Stopping rule of the adaptive variants ([PT] Significância e Alegações, "Direções Futuras": the
 * solver work chosen per block).  Reading: a block stops before step k >= 1 as soon as its monitor
 * is <= tol and keeps its iterates; tol < 0 never stops.  orc_ndb_until returns the steps run. */
int orc_ndb_until(int n, const double* M, int T, double tol, double* Y, double* Z, double* monitor) {
  const size_t nn = (size_t)n * n;
  double* P = (double*)malloc(sizeof(double) * nn);
  double* S = (double*)malloc(sizeof(double) * nn);
  double* Yn = (double*)malloc(sizeof(double) * nn);
  double* Zn = (double*)malloc(sizeof(double) * nn);
  memcpy(Y, M, sizeof(double) * nn);
  set_identity(n, Z, 1.0);
  int k = 0;
  for (; k < T; ++k) {
    orc_matmul(n, Z, Y, P);
    const double m = dist_to_identity(n, P);
    if (monitor) monitor[k] = m;
    if (tol >= 0.0 && k >= 1 && m <= tol) break;
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) S[IDX(i, j, n)] = (i == j ? 1.5 : 0.0) - 0.5 * P[IDX(i, j, n)];
    orc_matmul(n, Y, S, Yn);
    orc_matmul(n, S, Z, Zn);
    memcpy(Y, Yn, sizeof(double) * nn);
    memcpy(Z, Zn, sizeof(double) * nn);
  }
  free(P);
  free(S);
  free(Yn);
  free(Zn);
  return k;
}

void orc_ndb(int n, const double* M, int T, double* Y, double* Z, double* monitor) {
  orc_ndb_until(n, M, T, -1.0, Y, Z, monitor);
}

/* c5: inverse fourth root by two NDB calls.  Reading: the first call on A_s = A/s gives
 * Y = A_s^{1/2}; the second call on that Y gives Z = (A_s^{1/2})^{-1/2} = A_s^{-1/4};
 * X = s^{-1/4} Z.  T1 and T2 count steps per call.  Optional outputs: sqrt_out = s^{1/2} Y
 * (the square root of A, the pages' by-product), monitor[0..T1+T2) as in orc_ndb. */
void orc_ndb_inverse_root_until(int n, const double* A, double s, int T1, int T2, double tol, double* X,
                                double* sqrt_out, double* monitor, int* steps) {
  const size_t nn = (size_t)n * n;
  double* As = (double*)malloc(sizeof(double) * nn);
  double* Y = (double*)malloc(sizeof(double) * nn);
  double* Z = (double*)malloc(sizeof(double) * nn);
  for (size_t e = 0; e < nn; ++e) As[e] = A[e] / s;
  const int s1 = orc_ndb_until(n, As, T1, tol, Y, Z, monitor);
  if (sqrt_out)
    for (size_t e = 0; e < nn; ++e) sqrt_out[e] = sqrt(s) * Y[e];
  memcpy(As, Y, sizeof(double) * nn);
  const int s2 = orc_ndb_until(n, As, T2, tol, Y, Z, monitor ? monitor + T1 : NULL);
  if (steps) {
    steps[0] = s1;
    steps[1] = s2;
  }
  const double u = pow(s, -0.25);
  for (size_t e = 0; e < nn; ++e) X[e] = u * Z[e];
  free(As);
  free(Y);
  free(Z);
}

void orc_ndb_inverse_root(int n, const double* A, double s, int T1, int T2, double* X, double* sqrt_out,
                          double* monitor) {
  orc_ndb_inverse_root_until(n, A, s, T1, T2, -1.0, X, sqrt_out, monitor, NULL);
}

/* ------------------------------------------------------------------------------------------------
 * NDB with binary16 iterates and an fp32-precision correction ([PT] Resultados Experimentais: NDB in
 * FP16/BF16 was found unstable; [PT] Significância e Alegações, "Direções Futuras": stabilising NDB
 * in lower precision with error correction is named as future work).  Reading: the products are
 * exact (fp32 accumulation on the GPU) and every stored iterate is rounded to binary16:
 *     M = h(A/s);  call(M, T): S = h(1.5 I - 0.5 M), Z = S, Y = h(M S);
 *                  for k = 1 .. T-1: S = h(1.5 I - 0.5 Z Y), Y = h(Y S), Z = h(S Z),
 * composed as for c5 (call 1 on M gives Y, call 2 on that Y gives Z), except that the last Z of
 * call 2 is kept unrounded.  Then up to `refine` guarded correction steps against the unrounded
 * A_s = A/s: the candidate is a Newton step for the inverse fourth root followed by symmetrisation,
 *     X_c = sym(X (5 I - X^4 A_s) / 4),   sym(W) = (W + W^T) / 2,
 * taken only if it lowers the residual ||X^4 A_s - I||_F; at the first candidate that does not, the
 * correction stops (the Newton step is not contractive for every spectrum).  X = s^{-1/4} X.
 * h() rounds to the storage format: binary16 (orc_round_binary16), or bfloat16
 * (orc_round_bfloat16) in orc_ndb_lowp_inverse_root with fmt = 2 (the pages name FP16 and BF16
 * NDB together).
 * ---------------------------------------------------------------------------------------------- */
static void round_all(int fmt, size_t nn, double* x) {
  for (size_t e = 0; e < nn; ++e) x[e] = round_fmt(fmt, x[e]);
}

/* one low-precision NDB call; *Yout / *Zout receive Y_T / Z_T (Z_T unrounded when keep_z_exact) */
static void ndb_half_call(int n, int fmt, const double* M, int T, int keep_z_exact, double* Y, double* Z) {
  const size_t nn = (size_t)n * n;
  double* S = (double*)malloc(sizeof(double) * nn);
  double* P = (double*)malloc(sizeof(double) * nn);
  double* T1 = (double*)malloc(sizeof(double) * nn);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) S[IDX(i, j, n)] = (i == j ? 1.5 : 0.0) - 0.5 * M[IDX(i, j, n)];
  round_all(fmt, nn, S);
  memcpy(Z, S, sizeof(double) * nn);
  orc_matmul(n, M, S, Y);
  round_all(fmt, nn, Y);
  for (int k = 1; k < T; ++k) {
    orc_matmul(n, Z, Y, P);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) S[IDX(i, j, n)] = (i == j ? 1.5 : 0.0) - 0.5 * P[IDX(i, j, n)];
    round_all(fmt, nn, S);
    orc_matmul(n, Y, S, T1);
    round_all(fmt, nn, T1);
    memcpy(Y, T1, sizeof(double) * nn);
    orc_matmul(n, S, Z, T1);
    if (!(keep_z_exact && k == T - 1)) round_all(fmt, nn, T1);
    memcpy(Z, T1, sizeof(double) * nn);
  }
  free(S);
  free(P);
  free(T1);
}

void orc_ndb_lowp_inverse_root(int n, const double* A, double s, int T1, int T2, int fmt, int refine, double* X) {
  const size_t nn = (size_t)n * n;
  double* As = (double*)malloc(sizeof(double) * nn);
  double* M = (double*)malloc(sizeof(double) * nn);
  double* Y = (double*)malloc(sizeof(double) * nn);
  double* Z = (double*)malloc(sizeof(double) * nn);
  double* X2 = (double*)malloc(sizeof(double) * nn);
  double* X4 = (double*)malloc(sizeof(double) * nn);
  double* Mr = (double*)malloc(sizeof(double) * nn);
  for (size_t e = 0; e < nn; ++e) As[e] = A[e] / s;
  for (size_t e = 0; e < nn; ++e) M[e] = round_fmt(fmt, As[e]);
  ndb_half_call(n, fmt, M, T1, 0, Y, Z);
  memcpy(M, Y, sizeof(double) * nn);
  ndb_half_call(n, fmt, M, T2, 1, Y, Z);
  /* T = (5I - X^4 A_s)/4 of the current X (in Mr) and its residual ||X^4 A_s - I|| = 4 ||T - I|| */
  double* Xc = (double*)malloc(sizeof(double) * nn);
  double* Tc = (double*)malloc(sizeof(double) * nn);
#define EVAL_T(Xin, Tout, rout)                                                                    \
  do {                                                                                             \
    orc_matmul(n, (Xin), (Xin), X2);                                                               \
    orc_matmul(n, X2, X2, X4);                                                                     \
    orc_matmul(n, X4, As, (Tout));                                                                 \
    for (int i = 0; i < n; ++i)                                                                    \
      for (int j = 0; j < n; ++j) (Tout)[IDX(i, j, n)] = ((i == j ? 5.0 : 0.0) - (Tout)[IDX(i, j, n)]) / 4.0; \
    (rout) = 4.0 * dist_to_identity(n, (Tout));                                                    \
  } while (0)
  double r_cur = 0.0, r_c = 0.0;
  if (refine > 0) EVAL_T(Z, Mr, r_cur);
  for (int r = 0; r < refine; ++r) {
    orc_matmul(n, Z, Mr, X2);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) Xc[IDX(i, j, n)] = 0.5 * (X2[IDX(i, j, n)] + X2[IDX(j, i, n)]);
    EVAL_T(Xc, Tc, r_c);
    if (!(r_c < r_cur)) break;
    memcpy(Z, Xc, sizeof(double) * nn);
    memcpy(Mr, Tc, sizeof(double) * nn);
    r_cur = r_c;
  }
#undef EVAL_T
  free(Xc);
  free(Tc);
  const double u = pow(s, -0.25);
  for (size_t e = 0; e < nn; ++e) X[e] = u * Z[e];
  free(As);
  free(M);
  free(Y);
  free(Z);
  free(X2);
  free(X4);
  free(Mr);
}

void orc_ndb_half_inverse_root(int n, const double* A, double s, int T1, int T2, int refine, double* X) {
  orc_ndb_lowp_inverse_root(n, A, s, T1, T2, 1, refine, X);
}

/* ------------------------------------------------------------------------------------------------
 * c6: Coupled-Newton iteration for the inverse p-th root, p = 4 ([PT] Definição do Problema,
 * item 2; [TG] body, "CN - Coupled Newton Iteration").
 * Reading: the coupled Newton iteration of Guo and Higham (2006) with c = 1, on A_s = A/s:
 *     X_0 = I, M_0 = A_s;   S = ((p+1) I - M_k) / p,  X_{k+1} = X_k S,  M_{k+1} = M_k S^p,
 * with S^4 formed as (S S)(S S).  X_T -> A_s^{-1/4}; X = s^{-1/4} X_T.
 * half_storage (a storage format: 0 exact, 1 binary16, 2 bfloat16) rounds every stored iterate
 * (S, S^2, S^4, M, X) and the input operand A_s to that format, modelling 2-byte operands with
 * exact accumulation.
 * monitor[k] (optional) = ||M_k - I||_F / sqrt(n), before step k.
 * ---------------------------------------------------------------------------------------------- */
int orc_cn_until(int n, const double* A, double s, int T, int half_storage, double tol, double* X,
                 double* monitor) {
  const size_t nn = (size_t)n * n;
  double* M = (double*)malloc(sizeof(double) * nn);
  double* S = (double*)malloc(sizeof(double) * nn);
  double* S2 = (double*)malloc(sizeof(double) * nn);
  double* S4 = (double*)malloc(sizeof(double) * nn);
  double* Xk = (double*)malloc(sizeof(double) * nn);
  double* tmp = (double*)malloc(sizeof(double) * nn);
#define STORE16(buf)                                                   \
  do {                                                                 \
    if (half_storage)                                                  \
      for (size_t e_ = 0; e_ < nn; ++e_) (buf)[e_] = round_fmt(half_storage, (buf)[e_]); \
  } while (0)
  for (size_t e = 0; e < nn; ++e) M[e] = A[e] / s;
  STORE16(M);
  set_identity(n, Xk, 1.0);
  int k = 0;
  for (; k < T; ++k) {
    const double m = dist_to_identity(n, M);
    if (monitor) monitor[k] = m;
    if (tol >= 0.0 && k >= 1 && m <= tol) break;  /* stopping rule as in orc_ndb_until */
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) S[IDX(i, j, n)] = ((i == j ? 5.0 : 0.0) - M[IDX(i, j, n)]) / 4.0;
    STORE16(S);
    orc_matmul(n, Xk, S, tmp);
    memcpy(Xk, tmp, sizeof(double) * nn);
    if (k + 1 < T) STORE16(Xk);
    orc_matmul(n, S, S, S2);
    STORE16(S2);
    orc_matmul(n, S2, S2, S4);
    STORE16(S4);
    orc_matmul(n, M, S4, tmp);
    memcpy(M, tmp, sizeof(double) * nn);
    STORE16(M);
  }
#undef STORE16
  const double u = pow(s, -0.25);
  for (size_t e = 0; e < nn; ++e) X[e] = u * Xk[e];
  free(M);
  free(S);
  free(S2);
  free(S4);
  free(Xk);
  free(tmp);
  return k;
}

void orc_cn_inverse_root(int n, const double* A, double s, int T, int half_storage, double* X, double* monitor) {
  orc_cn_until(n, A, s, T, half_storage, -1.0, X, monitor);
}

/* ------------------------------------------------------------------------------------------------
 * c7: Chebyshev approximation evaluated by Clenshaw's recurrence ([PT] Metodologia, item 2,
 * "Aproximações de Polinômios de Chebyshev": Clenshaw's algorithm approximates the matrix power).
 * Reading: the degree-d interpolant of f(x) = x^expo at the d+1 Chebyshev points of the first kind
 * mapped to [lo, hi]:
 *     t_j = cos(pi (j + 1/2) / (d + 1)),  x_j = ((hi - lo) t_j + hi + lo) / 2,   j = 0..d,
 *     c_k = 2/(d+1) sum_j f(x_j) cos(pi k (j + 1/2) / (d + 1)),  then c_0 <- c_0 / 2,
 * so that p(x) = sum_k c_k T_k(t(x)) with t(x) = (2x - lo - hi) / (hi - lo).
 * ---------------------------------------------------------------------------------------------- */
void orc_cheb_coeffs(int d, double lo, double hi, double expo, double* c) {
  const double pi = acos(-1.0);
  for (int k = 0; k <= d; ++k) {
    double acc = 0.0;
    for (int j = 0; j <= d; ++j) {
      const double tj = cos(pi * (j + 0.5) / (d + 1));
      const double xj = ((hi - lo) * tj + hi + lo) / 2.0;
      acc += pow(xj, expo) * cos(pi * k * (j + 0.5) / (d + 1));
    }
    c[k] = 2.0 * acc / (d + 1);
  }
  c[0] /= 2.0;
}

/* P = sum_k c_k T_k(That) for the n x n matrix As, That = (2 As - (lo + hi) I) / (hi - lo), by
 * Clenshaw's recurrence: b_{d+1} = b_{d+2} = 0, b_k = c_k I + 2 That b_{k+1} - b_{k+2} for
 * k = d..1, P = c_0 I + That b_1 - b_2. */
void orc_clenshaw(int n, const double* As, int d, const double* c, double lo, double hi, double* P) {
  const size_t nn = (size_t)n * n;
  double* Th = (double*)malloc(sizeof(double) * nn);
  double* b1 = (double*)calloc(nn, sizeof(double)); /* b_{k+1} */
  double* b2 = (double*)calloc(nn, sizeof(double)); /* b_{k+2} */
  double* bk = (double*)malloc(sizeof(double) * nn);
  double* tb = (double*)malloc(sizeof(double) * nn);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      Th[IDX(i, j, n)] = (2.0 * As[IDX(i, j, n)] - (i == j ? lo + hi : 0.0)) / (hi - lo);
  for (int k = d; k >= 1; --k) {
    orc_matmul(n, Th, b1, tb);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j)
        bk[IDX(i, j, n)] = (i == j ? c[k] : 0.0) + 2.0 * tb[IDX(i, j, n)] - b2[IDX(i, j, n)];
    memcpy(b2, b1, sizeof(double) * nn);
    memcpy(b1, bk, sizeof(double) * nn);
  }
  orc_matmul(n, Th, b1, tb);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) P[IDX(i, j, n)] = (i == j ? c[0] : 0.0) + tb[IDX(i, j, n)] - b2[IDX(i, j, n)];
  free(Th);
  free(b1);
  free(b2);
  free(bk);
  free(tb);
}

/* Inverse fourth root by a degree-d Chebyshev interpolant of x^{-1/4} on [lo, hi] applied to
 * A_s = A/s; X = s^{-1/4} p(A_s). */
void orc_cheb_inverse_root(int n, const double* A, double s, int d, double lo, double hi, double* X) {
  const size_t nn = (size_t)n * n;
  double* c = (double*)malloc(sizeof(double) * (d + 1));
  double* As = (double*)malloc(sizeof(double) * nn);
  orc_cheb_coeffs(d, lo, hi, -0.25, c);
  for (size_t e = 0; e < nn; ++e) As[e] = A[e] / s;
  orc_clenshaw(n, As, d, c, lo, hi, X);
  const double u = pow(s, -0.25);
  for (size_t e = 0; e < nn; ++e) X[e] *= u;
  free(c);
  free(As);
}

/* ------------------------------------------------------------------------------------------------
 * Per-block interval bottom and solver choice ([PT] Significância e Alegações, "Direções Futuras":
 * the solver and its work chosen per block from the block's conditioning; no method is given).
 * ---------------------------------------------------------------------------------------------- */

/* Estimate of lambda_min(A) from above: the Multi-Power-Iteration of c3 run on C = sigma I - A
 * (same normalisation, Rayleigh quotients from the last product, max over columns), returning
 * sigma - max_j mu_j(C).  mu receives the k quotients of C. */
double orc_mpi_shifted(int n, const double* A, double sigma, int k, int T, const double* V0, double* mu) {
  const size_t nn = (size_t)n * n;
  double* C = (double*)malloc(sizeof(double) * nn);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) C[IDX(i, j, n)] = (i == j ? sigma : 0.0) - A[IDX(i, j, n)];
  const double top = orc_mpi(n, C, k, T, V0, mu);
  free(C);
  return sigma - top;
}

/* Residual of X as an inverse fourth root of A seen through k probe vectors: with v_j the
 * normalised columns of V0 (B x k, row-major) and E = X^4 A - I,
 *     r^2 = (1/k) sum_j ||E v_j||^2,
 * E v_j formed as X (X (X (X (A v_j)))) - v_j, one matrix-vector product at a time. */
double orc_residual_probe(int n, const double* A, const double* X, int k, const double* V0) {
  double* v = (double*)malloc(sizeof(double) * n);
  double* y = (double*)malloc(sizeof(double) * n);
  double* z = (double*)malloc(sizeof(double) * n);
  double total = 0.0;
  for (int j = 0; j < k; ++j) {
    double nrm = 0.0;
    for (int i = 0; i < n; ++i) nrm += V0[IDX(i, j, k)] * V0[IDX(i, j, k)];
    nrm = sqrt(nrm);
    for (int i = 0; i < n; ++i) v[i] = V0[IDX(i, j, k)] / nrm;
    for (int i = 0; i < n; ++i) {  /* y = A v */
      double acc = 0.0;
      for (int l = 0; l < n; ++l) acc += A[IDX(i, l, n)] * v[l];
      y[i] = acc;
    }
    for (int rep = 0; rep < 4; ++rep) {  /* y = X y, four times */
      for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int l = 0; l < n; ++l) acc += X[IDX(i, l, n)] * y[l];
        z[i] = acc;
      }
      memcpy(y, z, sizeof(double) * n);
    }
    for (int i = 0; i < n; ++i) total += (y[i] - v[i]) * (y[i] - v[i]);
  }
  free(v);
  free(y);
  free(z);
  return sqrt(total / k);
}

/* One block of the routed inverse root.  Reading of the pages' per-block solver choice:
 *   lam = orc_mpi_shifted(A, hi s) when est_steps > 0 (else no estimate),
 *   lo  = max(floor, lam / 2) / s,
 *   X   = degree-d Chebyshev inverse root of A on [lo, hi] in units of A/s (c7);
 *   r   = orc_residual_probe(A, X, V0);
 *   when r > tol (or r is NaN): X = coupled Newton p = 4 (c6) with the stopping rule of
 *   orc_cn_until at tol / 2 and at most cn_iters steps, and route = 1; else route = 0.
 * lam_out, r_out receive lam (NaN without an estimate) and r.  Returns route. */
int orc_routed_inverse_root(int n, const double* A, double s, int d, double floor, double hi, int k,
                            int est_steps, const double* V0, double tol, int cn_iters, double* X, double* lam_out,
                            double* r_out) {
  double lam = NAN;
  double lo_abs = floor;
  if (est_steps > 0) {
    double* mu = (double*)malloc(sizeof(double) * k);
    lam = orc_mpi_shifted(n, A, hi * s, k, est_steps, V0, mu);
    free(mu);
    if (0.5 * lam > lo_abs) lo_abs = 0.5 * lam;
  }
  orc_cheb_inverse_root(n, A, s, d, lo_abs / s, hi, X);
  const double r = orc_residual_probe(n, A, X, k, V0);
  int route = 0;
  if (!(r <= tol)) {
    orc_cn_until(n, A, s, cn_iters, 0, 0.5 * tol, X, NULL);
    route = 1;
  }
  if (lam_out) *lam_out = lam;
  if (r_out) *r_out = r;
  return route;
}

/* ------------------------------------------------------------------------------------------------
 * c8: Shampoo statistics update ([TG] body: two matrices L and R are kept from products of the
 * gradient, and their -1/4 power is taken).  Reading: exponential moving average
 *     L <- beta L + (1 - beta) G G^T,   R <- beta R + (1 - beta) G^T G,   in place.
 * ---------------------------------------------------------------------------------------------- */
void orc_update_stats(int n, const double* G, double beta, double* L, double* R) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      double ggt = 0.0, gtg = 0.0;
      for (int k = 0; k < n; ++k) {
        ggt += G[IDX(i, k, n)] * G[IDX(j, k, n)];
        gtg += G[IDX(k, i, n)] * G[IDX(k, j, n)];
      }
      L[IDX(i, j, n)] = beta * L[IDX(i, j, n)] + (1.0 - beta) * ggt;
      R[IDX(i, j, n)] = beta * R[IDX(i, j, n)] + (1.0 - beta) * gtg;
    }
}

/* 1-D parameters: a vector piece g of length n keeps L <- beta L + (1 - beta) g g^T, and its update is
 * L^{-1/2} g (Shampoo's exponent -1/(2k) for an order-k tensor, k = 1; the pages treat matrices only). */
void orc_update_stats_vec(int n, const double* g, double beta, double* L) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) L[IDX(i, j, n)] = beta * L[IDX(i, j, n)] + (1.0 - beta) * g[i] * g[j];
}

/* u = X g. */
void orc_apply_vec(int n, const double* X, const double* g, double* u) {
  for (int i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += X[IDX(i, j, n)] * g[j];
    u[i] = acc;
  }
}

/* Inverse square root by one NDB call (c4) on A/s: Z -> (A/s)^{-1/2}, X = s^{-1/2} Z. */
void orc_ndb_inverse_sqrt(int n, const double* A, double s, int T, double* X) {
  const size_t nn = (size_t)n * n;
  double* M = (double*)malloc(sizeof(double) * nn);
  double* Y = (double*)malloc(sizeof(double) * nn);
  double* mon = (double*)malloc(sizeof(double) * (T > 0 ? T : 1));
  for (size_t e = 0; e < nn; ++e) M[e] = A[e] / s;
  orc_ndb(n, M, T, Y, X, mon);
  const double r = 1.0 / sqrt(s);
  for (size_t e = 0; e < nn; ++e) X[e] *= r;
  free(M);
  free(Y);
  free(mon);
}

/* c9: preconditioned update U = L^{-1/4} G R^{-1/4} = (XL G) XR ([TG] body). */
void orc_apply(int n, const double* XL, const double* G, const double* XR, double* U) {
  double* T = (double*)malloc(sizeof(double) * (size_t)n * n);
  orc_matmul(n, XL, G, T);
  orc_matmul(n, T, XR, U);
  free(T);
}
