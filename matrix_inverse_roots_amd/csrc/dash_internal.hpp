// dash_internal.hpp -- internal declarations shared by the HIP translation units of libdash.
//
// Everything here is private to the library; the public surface is include/dash.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/dash.h"

namespace dash {

// ------------------------------------------------------------------------------------------------
// Per-block coefficient table.  One row of COEF_STRIDE floats per block, computed on the device
// from the scale s_i so that the host never reads s (no synchronisation).
// ------------------------------------------------------------------------------------------------
enum CoefIdx : int {
  CO_R1 = 0,    // 1 / s
  CO_R2 = 1,    // 1 / s^2
  CO_U = 2,     // s^{-1/4}        (final unscaling of an inverse fourth root)
  CO_SQ = 3,    // s^{1/2}         (unscaling of a square root)
  CO_R1U = 4,   // s^{-1} s^{-1/4}
  CO_P2 = 5,    // 2^-e: binary16 prescale of the power iteration
  CO_P2INV = 6, // 2^e
  CO_S = 7,     // s
  CO_RSQ = 8,   // s^{-1/2}        (unscaling of an inverse square root)
  CO_NONE = -1
};
constexpr int COEF_STRIDE = 10;

// Epilogue of a batched product acc = X_b Y_b (fp32 accumulation):
//   D  = alpha_b acc + beta_b C + delta_b E + gamma_b I        (C, E optional fp32 stacks)
//   D2 = alpha2_b acc + gamma2_b I                             (optional second output)
// with every coefficient = scalar * (idx >= 0 ? coef[b * COEF_STRIDE + idx] : 1).
// monitor (optional): monitor[b * mon_stride] += mon_mul * sum over the block of (D - I)^2
//   (accumulated with atomics; the caller zero-fills it and takes sqrt/ sqrt(B) afterwards).
// status (optional): status[b] |= 2 when D or D2 holds a non-finite value.
// fold_c (fp32 triangle-only NN products whose C is their right operand Y, i.e. Clenshaw's
// b_{k+1}): D = alpha_b (acc + c_over_a_b C) + delta_b E + gamma_b I, with C added from the staged
// (and possibly mapped) Y slices inside the product and E loaded during its last k-slice.  E is
// required, except in a launch that maps Y, which takes none.  c_over_a_b = c_over_a * coef[ic]
// must equal beta_b / alpha_b, and beta/ib are then unused.
struct Epilogue {
  float alpha = 1.f, beta = 0.f, delta = 0.f, gamma = 0.f, alpha2 = 0.f, gamma2 = 0.f;
  int8_t ia = CO_NONE, ib = CO_NONE, id = CO_NONE, ig = CO_NONE, ia2 = CO_NONE, ig2 = CO_NONE;
  bool fold_c = false;
  float c_over_a = 0.f;
  int8_t ic = CO_NONE;
  const float* coef = nullptr;
  float* monitor = nullptr;
  int32_t mon_stride = 0;
  float mon_mul = 1.f;
  int32_t* status = nullptr;
};

// One batched product over N blocks: D_b = epi(X_b Y_b).  X/Y element type is `in_prec`,
// D/D2 element type is `out_prec`; C/E are fp32.  Stride between blocks: B*B elements.
// map_x / map_y: the operand enters the product as a Z + g I, a = map_a * coef[map_ia] and
// g = map_g * coef[map_ig] (the fp32 kernel; binary16 kernels take map_g alone), formed while it is
// staged.  Binary16 operands (map_ia unused): map_a must be a power of two (each element
// is then the exact value rounded once to binary16).  fp32 operands: only map_y, in the Clenshaw
// launches (fold_c), one fma per element.
// freeze (optional, [N]; fp32 full NN products and binary16 triangle-only NN products): a block b
// with freeze[b] != 0 has stopped
// iterating.  Its product is not computed: pass = 0 writes nothing, pass = 1 / 2 writes the
// epilogue applied to X_b / Y_b in place of X_b Y_b (the iterate goes through unchanged).
// freeze[b] == 2 (fp32 kernel): the block is excluded from the call and nothing is written for it
// in any pass (a block another solver handles).
struct Product {
  const void* X = nullptr;
  const void* Y = nullptr;
  const float* C = nullptr;
  const float* E = nullptr;
  void* D = nullptr;
  void* D2 = nullptr;
  bool map_x = false, map_y = false;
  float map_a = 0.f, map_g = 0.f;
  int8_t map_ia = CO_NONE, map_ig = CO_NONE;
  const int32_t* freeze = nullptr;
  int8_t pass = 0;
  // two-piece binary16 products (DASH_FP32_SPLIT16): per-block bounds on |X| and |Y|, each the
  // largest of amax_*_parts values per block ([N][parts]), and where each wave of the launch
  // stores the largest |D| it wrote ([N][tiles][8]: one value per wave of every tile of the block,
  // every one written; null: not gathered)
  const float* amax_x = nullptr;
  const float* amax_y = nullptr;
  int amax_x_parts = 1, amax_y_parts = 1;
  float* amax_d = nullptr;
};

enum class Trans { NN, NT, TN };  // NT: Y read transposed, TN: X read transposed

// Enqueue one or two batched products sharing shape, precision and epilogue scalars (two problems
// in one launch fill the GPU better).  sym: compute only the upper-triangle tiles and mirror them
// (exactly symmetric output; C and E read from the upper triangle; no second output D2).  y_sym: every right operand Y is
// exactly symmetric (Y^T == Y bitwise), so binary16 kernels may read its columns as rows.
hipError_t launch_gemm(const Product* probs, int nprob, int64_t N, int B, dash_prec in_prec, dash_prec out_prec,
                       Trans trans, bool sym, const Epilogue& epi, hipStream_t stream, bool y_sym = false);

// D_b = a_b X_b + g_b I (and optionally D2_b = a2_b X_b + g2_b I), elementwise; X is fp32 or
// binary16 (x_prec).  X may be NULL (then D = g_b I).  Output precisions per output.  Optional
// monitor/status as above (monitor from D).
struct Affine {
  const void* X = nullptr;
  dash_prec x_prec = DASH_FP32;
  void* D = nullptr;
  dash_prec d_prec = DASH_FP32;
  float a = 0.f, g = 0.f;
  int8_t ia = CO_NONE, ig = CO_NONE;
  void* D2 = nullptr;
  dash_prec d2_prec = DASH_FP32;
  float a2 = 0.f, g2 = 0.f;
  int8_t ia2 = CO_NONE, ig2 = CO_NONE;
  const float* coef = nullptr;
  float* monitor = nullptr;
  int32_t mon_stride = 0;
  float mon_mul = 1.f;
  int32_t* status = nullptr;
};
hipError_t launch_affine(const Affine& op, int64_t N, int B, hipStream_t stream);
// The same map applied to the symmetric matrix built from the upper triangle of X (fp32 X, no
// status): D and D2 come out exactly symmetric.
hipError_t launch_sym_affine(const Affine& op, int64_t N, int B, hipStream_t stream);

// coef[b] from s[b]; status[b] bit 0 when s_b is not finite or not > 0 (all coefficients NaN).
hipError_t launch_coef(const float* s, int64_t N, float* coef, int32_t* status, hipStream_t stream);

// Fill n floats / int32 with a value (a kernel, never a memset node).
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);
// out[b] = max_ij |A_b[i][j]| (NaN elements passed over)
hipError_t launch_block_amax(const float* A, int64_t N, int B, float* out, hipStream_t stream);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);
// monitor[i] <- sqrt(monitor[i]) / sqrt(B)
hipError_t launch_monitor_finish(float* monitor, int64_t n, int B, hipStream_t stream);
// Stopping rule of the adaptive solvers.  Reset: freeze[b] = 0 and steps[b * steps_stride] = T
// (steps optional).  Update, after the launch that completed monitor column `col` (a sum of
// squares, before launch_monitor_finish): a block not yet frozen whose sqrt(sum)/sqrt(B) <= tol is
// frozen and steps[b * steps_stride] = step.
hipError_t launch_freeze_reset(int32_t* freeze, int32_t* steps, int steps_stride, int T, int64_t N,
                               hipStream_t stream);
// Guarded correction step (binary16 NDB): per block, take the candidate src[b] into dst[b] when its
// residual (monitor column q + 1) is below the current one (column q), else stop the block
// (freeze[b] = 1).  accept: [N] scratch.
hipError_t launch_accept(const float* mon, int mon_stride, int q, int32_t* freeze, int32_t* accept, const float* src,
                         float* dst, int64_t N, int B, hipStream_t stream);
hipError_t launch_freeze_update(const float* monitor, int mon_stride, int col, int B, float tol, int32_t* freeze,
                                int32_t* steps, int steps_stride, int step, int64_t N, hipStream_t stream);

// Chebyshev/Clenshaw plan, computed on the device per block: the interval [lo_b, hi] of x = A_b/s_b
// (lo_b = lo_rel when lo_rel > 0, else max(floor, theta lam[b]) / s_b), the degree-d interpolation
// coefficients of x^{-1/4} on it (fp64), and for every product launch q = 0 .. P-1 (P = max(1, d-1),
// in launch order) a row of epilogue coefficients tab[(q N + b) COEF_STRIDE + CS_*], each already
// multiplied by the s-dependent factor of the coefficient table.  A block whose interval is not
// 0 < lo_b < hi (or whose coefficients are not finite) gets NaN rows and status bit 0.
enum ChebSlot : int { CS_ALPHA = 0, CS_BETA = 1, CS_GAMMA = 2, CS_DELTA = 3, CS_COVERA = 4, CS_MAPA = 5, CS_MAPG = 6 };
constexpr int CHEB_MAX_DEGREE = 64;
struct ChebPlan {
  int64_t N = 0;
  int d = 0;
  bool split_first = false;  // first product in the split kernel's (alpha a1/s)(A + c I) A form
  const float* s = nullptr;
  const float* coef = nullptr;  // launch_coef's table
  double lo_rel = 0.0;
  double floor = 0.0;
  const float* lam = nullptr;
  float theta = 1.f;
  double hi = 1.0;
  float* tab = nullptr;      // [P, N, COEF_STRIDE]
  float* lo_out = nullptr;   // optional [N]
  int32_t* status = nullptr; // optional [N]
};
hipError_t launch_cheb_plan(const ChebPlan& p, hipStream_t stream);

// Routing of a two-solver call: route[b] = 1 (second solver) when r[b] > tol or r[b] is NaN, else
// 0; freeze[b] = route[b] ? 0 : 2 (blocks the second solver must leave alone).
hipError_t launch_route(const float* r, float tol, int64_t N, int32_t* route, int32_t* freeze, hipStream_t stream);
// dst[b] = src[b] where route[b] != 0 (per-block int32 select).
hipError_t launch_select_i32(const int32_t* src, const int32_t* route, int32_t* dst, int64_t N, hipStream_t stream);

// Scaling kernels.
hipError_t launch_frobenius(const float* A, int64_t N, int B, float* s, hipStream_t stream);
struct PowerPlan {
  int64_t N;
  int B, k, steps;
  dash_prec prec;
  const float* A;
  const float* V0;   // [B, k], or null: the pool drawn from seed (launch_start_pool's values)
  uint64_t seed = 0;
  float* s;
  // workspace pieces
  float* W[2];       // [N, B, 32] fp32 iterates
  float* part[2];    // [N, B/128, 3, 32] partial column sums
  float* V0p;        // [B, 32] normalised start vectors, zero columns from k on
  float* coef;       // [N, COEF_STRIDE] (prescale for binary16)
  _Float16* Ah;      // [N, B, B] binary16 operand (prec == DASH_FP16)
  // shifted iteration (fp32 only): when shift_s is set, each step forms W = sigma_b V - A V with
  // sigma_b = shift_mul * shift_s[b], and the result is s[b] = sigma_b - max_j mu_j (the smallest
  // eigenvalue estimate of A_b from the largest Rayleigh quotient of sigma_b I - A_b)
  const float* shift_s = nullptr;
  float shift_mul = 0.f;
};
hipError_t launch_power_iteration(const PowerPlan& plan, hipStream_t stream);
// coef[b][CO_P2] = 2^-e, coef[b][CO_P2INV] = 2^e with e = ceil(log2 max_j A_b[j][j]) (0, 0 when that
// maximum is not finite and > 0): the largest diagonal entry maps into (1/2, 1]
hipError_t launch_half_prescale(const float* A, int64_t N, int B, float* coef, hipStream_t stream);
// Stochastic residual: r[b] = sqrt(mean_{j<k} ||(X_b^4 A_b - I) v_j||^2) over the k normalised
// start vectors v_j (the columns of V0[B,k]), by five fp32 block-times-vectors passes (A, then X four
// times).  Workspace pieces as for the power iteration (W, part, V0p).
struct ProbePlan {
  int64_t N;
  int B, k;
  const float* A;
  const float* X;
  const float* V0;
  uint64_t seed = 0;
  float* r;
  float* W[2];
  float* part[2];
  float* V0p;
};
hipError_t launch_residual_probe(const ProbePlan& plan, hipStream_t stream);
// The start pool V0[e], e < n, drawn from seed (three SplitMix64 outputs per element, see scale.hip).
hipError_t launch_start_pool(uint64_t seed, int64_t n, float* V0, hipStream_t stream);
size_t power_workspace_bytes(int64_t N, int B, dash_prec prec);

// Eigendecomposition-based inverse fourth root (two-sided block Jacobi).  launch_jacobi runs up
// to max_sweeps sweeps on the matrices A (diagonalised in place), applying every rotation to V
// too.  Pass 0 starts the per-matrix sweep count, a later pass adds to it.  launch_evd_finish reads
// the eigenvalues w = diag(A) and writes Y = V diag(w^{-1/8}) (Y may be V).
struct JacobiPlan {
  int64_t N;
  int B, max_sweeps, pass;
  float tol;
  float* A;
  float* V;
  float* R;         // [N, B/64, 64, 64]
  int32_t* rot;     // [N, B/64]
  float* rsc = nullptr;  // with half: [N, B/64] power-of-two scales of the stored R - I
  int32_t* flags;   // [N, 8]
  bool half = false;            // update products as corrections M (R - I) from binary16 operands (R then
                                // holds (R - I)^T in binary16, scaled per pair by 1/rsc)
  bool pair_f32 = false;        // pair sub-problems solved in fp32 instead of fp64 (a pass that a refinement
                                // pass follows)
  const float* coef = nullptr;  // with half: per-block prescale (CO_P2, CO_P2INV), from launch_half_prescale
};
hipError_t launch_jacobi(const JacobiPlan& plan, hipStream_t stream);
struct EvdFinish {
  int64_t N;
  int B;
  const float* A;
  const float* V;
  float* Y;
  float* scale;     // [N, B]
  const int32_t* flags;
  float* eigvals;   // optional [N,B]
  int32_t* sweeps;  // optional [N]
  int32_t* status;  // optional [N]
};
hipError_t launch_evd_finish(const EvdFinish& f, hipStream_t stream);
hipError_t launch_identity(float* V, int64_t N, int B, hipStream_t stream);
size_t evd_workspace_bytes(int64_t N, int B);

// Stack / unstack n weights: the ceil(rows/B) x ceil(cols/B) tiles of each, in order, into
// consecutive blocks of `stack` (to_stack) or back out of it; the part of an edge tile outside the
// weight is zero in the stack and not written back.  One launch per COPY_GROUP weights.
constexpr int COPY_GROUP = 32;
struct CopyGroup {
  float* ptr[COPY_GROUP];
  int64_t ld[COPY_GROUP];
  int64_t rows[COPY_GROUP], cols[COPY_GROUP];
  int64_t row_base[COPY_GROUP + 1];  // first stack row (tile * B + r) of weight i in this launch
  int32_t wg_base[COPY_GROUP + 1];   // first workgroup of weight i
  int32_t tiles_c[COPY_GROUP];       // tile columns of weight i
  int32_t n;
};
hipError_t launch_tile_copy(const dash_mat* w, int n, int B, float* stack, bool to_stack, hipStream_t stream);

// 1-D parameters (vec.hip): a vector's pieces of B (the last zero-padded) copied to or from a
// contiguous run of pieces; the rank-one statistic update L_p <- beta L_p + (1 - beta) g_p g_p^T;
// u_p = X_p g_p.
hipError_t launch_vec_copy(float* v, int64_t len, float* pieces, int B, bool to_pieces, hipStream_t stream);
hipError_t launch_vec_stats(const float* g, int64_t P, int B, float beta, float* L, hipStream_t stream);
hipError_t launch_vec_apply(const float* X, const float* g, int64_t P, int B, float* u, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// dash_scale's argument checks short of the workspace (DASH_OK or the status dash_scale returns).
dash_status scale_args_check(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                             int32_t steps, const float* V0, const float* s);

}  // namespace dash
