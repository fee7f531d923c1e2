/*
 * dash.h -- C ABI of the MI355X (gfx950) batched inverse-fourth-root library.
 *
 * The library computes, for a stack of N independent symmetric positive-definite B x B blocks held
 * as one (N, B, B) tensor, the inverse fourth root A^{-1/4} that Shampoo needs, plus the steps
 * around it: stacking weight gradients into B x B tiles, the L/R statistic update, spectral
 * scaling, and applying the preconditioned update L^{-1/4} G R^{-1/4}.
 *
 * Pages cited (by title and section):
 *   [PT] "Resumo Técnico: DASH – Shampoo Mais Rápido via Pré-condicionamento de Blocos em Lote e
 *        Solvers de Raiz Inversa Eficientes" (gist.science/pt/paper/2602.02016)
 *   [TG] quant_prune_distill post 646 (tgviewer.app), commentary on DASH
 *   [AB] arxivdaily.com/papers/2602.02016, English abstract
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless marked [host].  Matrices are contiguous row-major fp32
 *   (fp16 appears only inside the library), 16-byte aligned; a stack of N blocks is N*B*B floats
 *   with block i at offset i*B*B.
 * - B % 64 == 0 and 64 <= B <= 8192; N >= 1.
 * - Ownership: the caller allocates and owns every buffer.  The library never allocates device
 *   memory, never synchronises the device or the stream and keeps no mutable global state.
 *   Scratch memory is the caller's `ws` of `ws_bytes` bytes (256-byte aligned), sized by
 *   dash_workspace_size(); its contents are undefined on return.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 * - Errors: argument, shape and workspace errors are detected on the host before anything is
 *   enqueued (nothing is launched); DASH_ERR_DEVICE reports a failed launch.  Numerical trouble
 *   never synchronises: per-block problems are reported in the optional `status[N]` array
 *   (bit 0: the scale s_i is not finite or not > 0, the block's output is NaN;
 *    bit 1: the block's output contains a non-finite value).  Other blocks are unaffected.
 * - Outputs must not alias inputs unless stated.
 */
#ifndef DASH_H_
#define DASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DASH_ABI_VERSION 1

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad count, parameter out of range */
  DASH_ERR_SHAPE = 2,       /* B not a multiple of 64 or out of range */
  DASH_ERR_WORKSPACE = 3,   /* ws too small or misaligned */
  DASH_ERR_UNSUPPORTED = 4, /* a valid request the library does not implement (e.g. p != 4) */
  DASH_ERR_DEVICE = 5       /* a HIP launch failed */
} dash_status;

/* operand precision; accumulation is fp32.  DASH_BF16 (bfloat16 operands: 8-bit significand, the
 * exponent range of fp32) is accepted by the half-precision solvers (dash_inverse_root_cn,
 * dash_inverse_root_ndb_lowp) and their workspace/flop queries; dash_scale takes DASH_FP32 or DASH_FP16.
 * DASH_FP32_SPLIT: fp32 operands, iterates and results, with each product formed on the bfloat16
 * matrix cores from an exact three-piece split of both operands (six piece products, fp32
 * accumulation; as accurate as an fp32 product); accepted by dash_inverse_root_cheb_prec,
 * dash_inverse_root_ndb_prec, dash_inverse_root_cn, dash_update_stats_prec and dash_apply_prec, by
 * dash_workspace_size (as DASH_FP32) and by dash_flops (DASH_OP_CHEB then counts 256-wide tiles
 * for degree >= 3 and B % 256 == 0).
 * DASH_FP32_SPLIT16: fp32 operands, iterates and results, with each product formed on the binary16
 * matrix cores from two-piece binary16 splits of both operands, each brought near 8 by a power of
 * two per block first (three piece products, fp32 accumulation; the pieces hold 22 of an fp32
 * value's 24 significant bits, and the product's error, measured against fp64, is that of an fp32
 * product); accepted by the Chebyshev solves (dash_inverse_root_cheb_prec,
 * dash_inverse_root_cheb_blocks and the Chebyshev step of dash_inverse_root_routed), by
 * dash_inverse_root_ndb_prec, dash_apply_prec and dash_update_stats_ws, and by dash_workspace_size
 * and dash_flops (as DASH_FP32_SPLIT). */
typedef enum { DASH_FP32 = 0, DASH_FP16 = 1, DASH_BF16 = 2, DASH_FP32_SPLIT = 3, DASH_FP32_SPLIT16 = 4 } dash_prec;

typedef enum { DASH_SCALE_FROBENIUS = 0, DASH_SCALE_POWER = 1 } dash_scaling;

typedef enum {
  DASH_OP_SCALE = 0,
  DASH_OP_NDB = 1,
  DASH_OP_CN = 2,
  DASH_OP_CHEB = 3,
  DASH_OP_APPLY = 4,
  DASH_OP_STATS = 5,
  DASH_OP_EVD = 6,
  DASH_OP_ROUTED = 7
} dash_op;

/* A row-major fp32 weight gradient (device memory): element (r, c) at ptr[r * ld + c]. */
typedef struct {
  float* ptr;
  int64_t rows, cols, ld;
} dash_mat;

/* A contiguous fp32 vector gradient (device memory) of len elements: a 1-D parameter. */
typedef struct {
  float* ptr;
  int64_t len;
} dash_vec;

/* Blockify: copy the B x B tiles of n weight gradients into G_stack, weight-major, then tile row,
 * then tile column ([PT] Metodologia, item 1: gradient blocks G_ij are stacked into an (N, B, B)
 * tensor so one batched call processes them all).
 * grads [host]: n descriptors, rows >= 1, cols >= 1, ld >= cols, ptr and ld*4 16-byte aligned.  A
 * weight gives ceil(rows/B) x ceil(cols/B) tiles; where its sides are not multiples of B, the part of
 * an edge tile outside the weight is zero.  G_stack: sum_w ceil(rows_w/B) ceil(cols_w/B) blocks.
 * (A zero-padded tile keeps zero rows/columns in its statistics; damping the L/R stack, e.g. an
 * initial eps I, keeps such blocks positive definite, and apply leaves the padding zero.) */
dash_status dash_stack(const dash_mat* grads, int32_t n, int32_t B, float* G_stack, void* stream);

/* Inverse of dash_stack: scatter the tiles of U_stack back into n weight-shaped outputs [host]
 * (the same shape rules; the padding of edge tiles is not written anywhere). */
dash_status dash_unstack(const float* U_stack, int32_t B, const dash_mat* outs, int32_t n, void* stream);

/* Shampoo statistics ([TG] body: L and R are kept from products of the gradient):
 *   L_t <- beta L_t + (1 - beta) G_t G_t^T,   R_t <- beta R_t + (1 - beta) G_t^T G_t,
 * for the NG gradient tiles G_stack[NG,B,B].  A is the stacked preconditioner statistic
 * [2*NG, B, B] updated IN PLACE: L blocks at [0, NG), R blocks at [NG, 2 NG) ([TG] body: the L and R
 * preconditioners are stacked into one tensor).  Only the upper triangle of each input block is
 * read; every output block is exactly symmetric.  0 <= beta <= 1. */
dash_status dash_update_stats(const float* G_stack, int64_t NG, int32_t B, float beta, float* A, void* stream);

/* dash_update_stats with the products' arithmetic chosen by prec: DASH_FP32 (the fp32 matrix cores;
 * the same as dash_update_stats) or DASH_FP32_SPLIT (both products formed from exact three-piece
 * bfloat16 splits of their fp32 operands on the bfloat16 matrix cores when B % 256 == 0; with
 * other B the fp32 matrix cores).  DASH_ERR_INVALID_ARG for any other prec. */
dash_status dash_update_stats_prec(const float* G_stack, int64_t NG, int32_t B, float beta, dash_prec prec, float* A,
                                   void* stream);

/* dash_update_stats_prec with a caller workspace, for DASH_FP32_SPLIT16: both products formed on the
 * binary16 matrix cores from two-piece binary16 splits of G, brought near 8 by a power of two per
 * tile (one pass over G_stack for each tile's bound, kept in ws; with B % 256 != 0 the fp32 matrix
 * cores and ws unused).  ws: dash_workspace_size(DASH_OP_STATS, NG, B, DASH_FP32_SPLIT16) bytes,
 * 256-byte aligned.  Any other prec: exactly dash_update_stats_prec (ws unused, may be NULL).
 * Arguments, results and errors otherwise as dash_update_stats_prec; DASH_ERR_WORKSPACE for a
 * missing or short ws where it is used. */
dash_status dash_update_stats_ws(const float* G_stack, int64_t NG, int32_t B, float beta, dash_prec prec, float* A,
                                 void* ws, size_t ws_bytes, void* stream);

/* Per-block scale s[N] ([PT] Definição do Problema, item 3, and Metodologia, item 2,
 * "Multi-Power-Iteration"; [TG] body: Rayleigh-quotient estimate of the spectral norm).
 *   DASH_SCALE_FROBENIUS: s_i = ||A_i||_F   (k, steps, V0, seed and prec ignored; ws may be NULL).
 *   DASH_SCALE_POWER:     k start vectors (columns of V0[B,k], shared by all blocks, 1 <= k <= 32)
 *     run `steps` >= 1 power-iteration steps in parallel: each step forms W = A_i V, the Rayleigh
 *     quotient of every column comes from the last step, each column is renormalised between
 *     steps, and s_i = max over columns.  prec == DASH_FP16 streams A_i in binary16 prescaled by
 *     2^-ceil(log2 max_j A_i[j][j]) and keeps V in binary16; accumulation stays fp32.
 *     prec == DASH_FP32_SPLIT (B % 128 == 0): each step's product is formed from exact three-piece
 *     bfloat16 splits of A_i and V on the bfloat16 matrix cores (six piece products, fp32
 *     accumulation), an fp32 product at a fraction of the fp32 matrix cores' time; other B run
 *     the DASH_FP32 step.  Workspace as DASH_FP32.
 *     V0 == NULL: the start pool is drawn on the device from `seed` (dash_start_vectors' values).
 * A block whose scale comes out non-finite or <= 0 is flagged later by the solver. */
dash_status dash_scale(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                       int32_t steps, const float* V0, uint64_t seed, float* s, void* ws, size_t ws_bytes,
                       void* stream);

/* The start pool V0[B,k] (row-major) that dash_scale draws from `seed` when it is given no V0.
 * Element e = i k + j is a centred sum of three uniforms from a SplitMix64 stream started at seed
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014: output n is
 * mix(seed + n 0x9E3779B97F4A7C15) with mix(z) = z ^ (z >> 30), times 0xBF58476D1CE4E5B9, ^ >> 27,
 * times 0x94D049BB133111EB, ^ >> 31): with u_q the top 22 bits of output 3e + q (q = 1, 2, 3),
 * V0[e] = (u_1 + u_2 + u_3 - 1.5 * 2^22) * 2^-22, in (-1.5, 1.5), exact in fp32.  The pages give no
 * distribution for the start vectors; any pool with a component along the top eigenvector serves.
 * 1 <= k <= 32. */
dash_status dash_start_vectors(int32_t B, int32_t k, uint64_t seed, float* V0, void* stream);

/* Inverse fourth root by two Newton-Denman-Beavers calls ([PT] Metodologia, item 2,
 * "Iteração de Newton-Denman-Beavers": one call gives the square root and the inverse square root;
 * the first step skips the products that the identity start makes redundant).
 * One call on M: Y_0 = M, Z_0 = I; per step P = Z Y, S = (3I - P)/2, Y <- Y S, Z <- S Z.
 * Call 1 runs iters1 steps on A_i / s_i giving Y ~ (A_i/s_i)^{1/2}; call 2 runs iters2 steps on
 * that Y giving Z ~ (A_i/s_i)^{-1/4}; X_i = s_i^{-1/4} Z.  3*iters - 3 products per call.
 * fp32 only.  iters1, iters2 >= 1.
 * sqrt_out: NULL or [N,B,B] receives s_i^{1/2} Y (the square root of A_i).
 * monitor:  NULL or [N, iters1 + iters2] receives ||P_k - I||_F / sqrt(B) per step.
 * status:   NULL or [N]. */
dash_status dash_inverse_root_ndb(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                  int32_t iters2, float* X, float* sqrt_out, float* monitor, int32_t* status,
                                  void* ws, size_t ws_bytes, void* stream);

/* dash_inverse_root_ndb with the products' arithmetic chosen by prec: DASH_FP32 (the fp32 matrix
 * cores; the same as dash_inverse_root_ndb), DASH_FP32_SPLIT (every product formed from exact
 * three-piece bfloat16 splits of its fp32 operands on the bfloat16 matrix cores, 256 x 256 tiles,
 * when B % 256 == 0; with other B the fp32 matrix cores) or DASH_FP32_SPLIT16 (the same tiles with
 * two-piece binary16 splits on the binary16 matrix cores, each operand scaled by a power of two per
 * block from a bound on its magnitude: a pass over A, over each elementwise result, and for each
 * product's result the per-wave maxima its launch stores).  Iterates stay fp32 and are never
 * symmetrised.  Same arguments, workspace and results contract otherwise; DASH_ERR_INVALID_ARG for
 * any other prec. */
dash_status dash_inverse_root_ndb_prec(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, dash_prec prec, float* X, float* sqrt_out, float* monitor,
                                       int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* NDB with binary16 iterates and an fp32 correction ([PT] Resultados Experimentais: NDB in FP16/BF16
 * was unstable in the authors' runs; [PT] Significância e Alegações, "Direções Futuras": stabilising
 * NDB in lower precision with error correction is named as future work).  The two composed NDB calls
 * run as in dash_inverse_root_ndb, with binary16 operands and fp32 accumulation, every stored
 * iterate rounded to binary16 once (M = A_i/s_i included; the second call's last Z is kept in fp32).
 * Then up to `refine` guarded correction steps against A_s = A_i/s_i in fp32: the candidate is a
 * Newton step for the inverse fourth root followed by symmetrisation, X_c = sym(X (5I - X^4 A_s)/4),
 * and a block takes it only if it lowers the block's residual ||X^4 A_s - I||_F (four fp32 products
 * per step and three to start); at its first candidate that does not, the block keeps its X and
 * stops correcting (the Newton step is contractive for well-conditioned blocks, kappa of order 10,
 * and diverges beyond).  X_i = s_i^{-1/4} X.  0 <= refine <= 16.  Workspace: dash_workspace_size(DASH_OP_NDB, ...,
 * DASH_FP16, ...).  Other arguments as for dash_inverse_root_ndb (no square-root output). */
dash_status dash_inverse_root_ndb_half(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, int32_t refine, float* X, float* monitor, int32_t* status,
                                       void* ws, size_t ws_bytes, void* stream);

/* The same with the iterates' 2-byte format chosen by prec: DASH_FP16 (binary16; identical to
 * dash_inverse_root_ndb_half) or DASH_BF16 (bfloat16: 8-bit significand, fp32's exponent range;
 * [PT] Resultados Experimentais name FP16/BF16 NDB together).  Products accumulate in fp32 and
 * every stored iterate is rounded to that format once.  Workspace: dash_workspace_size(DASH_OP_NDB,
 * ..., prec, ...).  Any other prec -> DASH_ERR_INVALID_ARG. */
dash_status dash_inverse_root_ndb_lowp(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, dash_prec prec, int32_t refine, float* X, float* monitor,
                                       int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* Inverse p-th root by the Coupled-Newton iteration, p = 4 ([PT] Definição do Problema, item 2;
 * [TG] body, "CN - Coupled Newton Iteration"; fp16 operands per [PT] Resultados Experimentais).
 * On M_0 = A_i / s_i, X_0 = I: S = (5I - M)/4, X <- X S, M <- M S^4 (S^4 = (S S)(S S));
 * X_i = s_i^{-1/4} X_iters.  4*iters - 4 products.  prec == DASH_FP16 (DASH_BF16) stores every
 * iterate in binary16 (bfloat16) and accumulates in fp32; X is always written in fp32.  p != 4 ->
 * DASH_ERR_UNSUPPORTED.  Only the upper triangle of A_i is read (the start terms are built from it,
 * mirrored).  With 2-byte operands every iterate (a polynomial in A_i) is kept exactly symmetric:
 * each product computes only its upper-triangle tiles and mirrors them, and X_i comes out exactly
 * symmetric.
 * fp32 runs full products, which keep the fp32 rounding floor lowest at high condition numbers.
 * prec == DASH_FP32_SPLIT: fp32 iterates with the products formed from exact three-piece bfloat16
 * splits on the bfloat16 matrix cores when B % 256 == 0, except the M S^4 launches that also write
 * S_{k+1} (fp32 cores; dash_inverse_root_cn_adaptive runs every product on the fp32 cores).
 * monitor: NULL or [N, iters] receives ||M_k - I||_F / sqrt(B) before step k. */
dash_status dash_inverse_root_cn(const float* A, const float* s, int64_t N, int32_t B, int32_t p, int32_t iters,
                                 dash_prec prec, float* X, float* monitor, int32_t* status, void* ws,
                                 size_t ws_bytes, void* stream);

/* Per-block adaptive variants of the two iterations ([PT] Significância e Alegações, "Direções
 * Futuras": the authors point to choosing the solver work per block from its conditioning).  Each
 * block stops iterating as soon as its own monitor is <= tol before a step k >= 1 (the first step
 * always runs): from then on its iterates pass through the remaining launches unchanged (no products
 * are computed for it) and its output is formed from them as usual.  A block whose monitor never
 * reaches tol runs all steps.  The monitor is the same as in the fixed-step calls: ||P_k - I|| for
 * NDB (each of the two calls stops on its own), ||M_k - I|| = ||X_k^4 A_s - I|| for CN, in
 * Frobenius norm over sqrt(B).
 * max_iters*: the step limits (as iters* above).  tol >= 0.  monitor is required ([N, max1 + max2]
 * for NDB, [N, max_iters] for CN); its entries after a block stopped are 0.
 * steps: NULL or [N, 2] (NDB: steps run by call 1 and call 2) / [N] (CN): the steps each block ran.
 * CN takes both precisions (with binary16 iterates a stopped block's X_k is the stored binary16
 * iterate, so its output carries one binary16 rounding more than a fixed run ending at step k).
 * Other arguments as above. */
dash_status dash_inverse_root_ndb_adaptive(const float* A, const float* s, int64_t N, int32_t B, int32_t max_iters1,
                                           int32_t max_iters2, float tol, float* X, float* sqrt_out, float* monitor,
                                           int32_t* steps, int32_t* status, void* ws, size_t ws_bytes,
                                           void* stream);
dash_status dash_inverse_root_cn_adaptive(const float* A, const float* s, int64_t N, int32_t B, int32_t p,
                                          int32_t max_iters, float tol, dash_prec prec, float* X, float* monitor,
                                          int32_t* steps, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* Inverse fourth root by a Chebyshev approximation evaluated with Clenshaw's recurrence
 * ([PT] Metodologia, item 2, "Aproximações de Polinômios de Chebyshev").  The degree-`degree`
 * interpolant p of x^{-1/4} at the Chebyshev points of the first kind on [lo, hi] is applied to
 * A_i / s_i; X_i = s_i^{-1/4} p(A_i / s_i).  degree - 1 products.  1 <= degree <= 64, 0 < lo < hi.
 * fp32 only.  A_i must be symmetric: the recurrence terms are polynomials in A_i, so each product
 * computes only its upper-triangle tiles and mirrors them; X_i comes out exactly symmetric. */
dash_status dash_inverse_root_cheb(const float* A, const float* s, int64_t N, int32_t B, int32_t degree, double lo,
                                   double hi, float* X, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* dash_inverse_root_cheb with the products' arithmetic chosen by prec: DASH_FP32 (the fp32 matrix
 * cores; the same as dash_inverse_root_cheb) or DASH_FP32_SPLIT (fp32 products formed from exact
 * three-piece bfloat16 splits on the bfloat16 matrix cores, 256 x 256 tiles, when B % 256 == 0 and
 * degree >= 3; the recurrence's C term enters as a shift of A's diagonal; with other B or degree 2
 * the fp32 matrix cores) or DASH_FP32_SPLIT16 (the same tiles and shapes with two-piece binary16
 * splits on the binary16 matrix cores: each product's operands are scaled by a power of two per
 * block from a bound on their magnitude, max |A_i| from a pass over the stack and max |b_k| from
 * the launch that wrote b_k; with other B or degree 2 the fp32 matrix cores).  Same arguments,
 * workspace and results contract otherwise; DASH_ERR_INVALID_ARG for any other prec. */
dash_status dash_inverse_root_cheb_prec(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                        double lo, double hi, dash_prec prec, float* X, int32_t* status, void* ws,
                                        size_t ws_bytes, void* stream);

/* dash_inverse_root_cheb_prec with an interval of its own for every block, derived on the device
 * (the host never reads s; [PT] Metodologia, item 2, "Aproximações de Polinômios de Chebyshev":
 * the pages give no interval, so the library takes it from what bounds each block's spectrum).
 * Block i's interval, in units of A_i / s_i, is [lo_i, hi] with
 *   lo_i = max(floor, theta * lam_min[i]) / s_i        (lam_min == NULL: lo_i = floor / s_i).
 * floor: an absolute lower bound of every block's spectrum (e.g. the damping eps I added to the
 *   statistics, times beta^t after t EMA updates), >= 0; > 0 when lam_min is NULL.
 * lam_min: NULL or [N] per-block estimates of the smallest eigenvalue (dash_spectrum_min), of which
 *   the fraction theta (0 < theta <= 1) is taken as the lower end.
 * hi: upper end relative to s_i, > 0 (e.g. 1.25 after power-iteration scaling, 1 after Frobenius).
 * The degree-`degree` interpolant of x^{-1/4} at the Chebyshev points of the first kind of block i's
 * interval is computed on the device in fp64.  lo_out: NULL or [N] receives lo_i.  A block whose
 * lo_i is not in (0, hi) gets status bit 0 and a NaN output (as for a bad s_i); so does a block whose
 * top Chebyshev coefficient underflows fp32 (degree near 64 on an interval with hi/lo_i near 1).
 * Products, precision, workspace (DASH_OP_CHEB) and results otherwise as dash_inverse_root_cheb_prec. */
dash_status dash_inverse_root_cheb_blocks(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                          double floor, const float* lam_min, float theta, double hi, dash_prec prec,
                                          float* X, float* lo_out, int32_t* status, void* ws, size_t ws_bytes,
                                          void* stream);

/* dash_scale without a caller workspace, for callers that cannot allocate device memory: code under
 * stream capture, serving loops and harnesses that forbid allocation.  Arguments and results as
 * dash_scale.  The power iteration's scratch lives in a device array owned by the library,
 * dash_noalloc_scratch_bytes() bytes (128 MiB) on every GPU the library runs on, held until the
 * process ends; the call allocates nothing.  A request whose scratch (dash_workspace_size of
 * DASH_OP_SCALE) exceeds it returns DASH_ERR_WORKSPACE before anything is enqueued (fp32: up to 488
 * blocks per call at B = 1024, 1954 at B = 256; binary16, which also holds the cast of A: 56 at 1024).  The current device must be the stream's.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (on two streams, or from two threads) race and
 * must be ordered by the caller.  The Frobenius scale needs no scratch and is passed through. */
dash_status dash_scale_noalloc(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                               int32_t steps, const float* V0, uint64_t seed, float* s, void* stream);
size_t dash_noalloc_scratch_bytes(void);

/* Estimate of every block's smallest eigenvalue, from above ([PT] Significância e Alegações,
 * "Direções Futuras": choosing the solver per block from its conditioning needs the bottom of each
 * block's spectrum; the pages name the largest eigenvalue's power iteration only, so this is the
 * same iteration on a shifted block).  With sigma_i = hi * s_i (hi > 0; s from dash_scale, so that
 * sigma_i >= lambda_max(A_i) when hi covers the scale's underestimate), `steps` power-iteration steps
 * with the k normalised start vectors V0[B,k] run on C_i = sigma_i I - A_i exactly as dash_scale's
 * (every column renormalised between steps, Rayleigh quotients from the last step) and
 *   lam_min[i] = sigma_i - max_j mu_j(C_i)   (>= lambda_min(A_i) up to rounding).
 * The estimate converges slowly where the bottom of the spectrum is dense (an excess of order
 * hi s_i / steps), and an isolated small eigenvalue may be missed; callers take a fraction of it
 * and check the result (dash_inverse_root_routed).  fp32, 1 <= k <= 32, steps >= 1.
 * Workspace: dash_workspace_size(DASH_OP_SCALE, N, B, DASH_FP32, k, ...). */
dash_status dash_spectrum_min(const float* A, const float* s, int64_t N, int32_t B, double hi, int32_t k,
                              int32_t steps, const float* V0, float* lam_min, void* ws, size_t ws_bytes,
                              void* stream);

/* Stochastic residual of a computed inverse fourth root: for the k normalised columns v_j of V0[B,k],
 *   r[i] = sqrt( (1/k) sum_j ||(X_i^4 A_i - I) v_j||^2 ),
 * formed by five fp32 block-times-vectors passes (A_i v, then X_i four times).  For v uniform on the
 * sphere E ||E v||^2 = ||E||_F^2 / B, so r[i] estimates the residual ||X_i^4 A_i - I||_F / sqrt(B) of
 * the accuracy gate (relative spread about sqrt(2/k)) at the cost of five reads of the stack.
 * 1 <= k <= 32.  Workspace: dash_workspace_size(DASH_OP_SCALE, N, B, DASH_FP32, k, ...). */
dash_status dash_residual_probe(const float* A, const float* X, int64_t N, int32_t B, int32_t k, const float* V0,
                                float* r, void* ws, size_t ws_bytes, void* stream);

/* Inverse fourth root with the solver chosen per block inside one call ([PT] Significância e
 * Alegações, "Direções Futuras": dynamic solver selection per block from its conditioning).
 *   1. lam_i = dash_spectrum_min estimate (est_steps steps; none when est_steps == 0);
 *   2. every block solved by degree-`degree` Chebyshev on its own interval
 *      [max(floor, lam_i / 2) / s_i, hi] (dash_inverse_root_cheb_blocks with theta = 1/2);
 *   3. the residual of every block estimated by dash_residual_probe with V0's k columns;
 *   4. the blocks whose estimate exceeds tol (or is NaN) solved again by coupled Newton p = 4 in fp32
 *      on the fp32 matrix cores, at most cn_iters steps, each block stopping once its monitor
 *      ||M_k - I|| / sqrt(B) (its exact residual) is <= tol / 2; their X_i replaced.
 * Blocks the estimate makes well conditioned keep the tight interval's accuracy; ill-conditioned
 * blocks, or blocks whose bottom eigenvalue the estimate overshot, are caught by the probe.
 * floor >= 0 (> 0 when est_steps == 0), hi > 0, 1 <= k <= 32, 0 <= est_steps, tol > 0,
 * 2 <= cn_iters <= 64; prec DASH_FP32, DASH_FP32_SPLIT or DASH_FP32_SPLIT16 (the Chebyshev
 * products).
 * lam_min: NULL or [N] receives the estimates (NaN when est_steps == 0); route: NULL or [N] receives
 * 0 (Chebyshev) or 1 (coupled Newton); resid: NULL or [N] receives the probe's residual estimate of
 * the final X_i (five more passes); status: as for the solvers, from the solver that wrote X_i.
 * Workspace: dash_workspace_size(DASH_OP_ROUTED, N, B, ...). */
dash_status dash_inverse_root_routed(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                     double floor, double hi, int32_t k, int32_t est_steps, const float* V0,
                                     float tol, int32_t cn_iters, dash_prec prec, float* X, float* lam_min,
                                     float* resid, int32_t* route, int32_t* status, void* ws, size_t ws_bytes,
                                     void* stream);

/* Inverse fourth root through an eigendecomposition A_i = Q diag(w) Q^T, X_i = Q diag(w^{-1/4}) Q^T
 * ([PT] Definição do Problema, item 2, and Resultados Experimentais: the eigendecomposition is the
 * root solver whose cost the iterations above avoid; [TG] body).  Batched two-sided block Jacobi in
 * fp32: the columns are cut into blocks of 32; each round pairs the blocks (circle schedule), runs
 * one sweep of scalar Jacobi on every 64 x 64 pair sub-problem and applies its rotation to A and to
 * the eigenvector estimate; a sweep is B/32 - 1 rounds.  Rotations are skipped where
 * |A_pq| <= 2^-22 sqrt(A_pp A_qq); a matrix is done after a sweep that rotates nothing, and later
 * sweeps skip it.  No scale s is needed (the method is scale-free).
 * refine = 1 adds a second pass: the eigenvector estimate Q is re-orthogonalised by one
 * Newton-Schulz step, H = Q^T A_i Q is formed from the input again, and the sweeps run on H.  This
 * removes the rounding the first pass accumulates in its working matrix, which dominates the
 * error at high condition numbers (four more products and a few sweeps on a nearly diagonal H).
 * Since the second pass starts from the input again, the first pass then solves its 64 x 64 pair
 * sub-problems in fp32; the second pass keeps fp64 ones.
 * A: [N,B,B], symmetric, read in full.  max_sweeps: 1 .. 100 per pass.  X: [N,B,B], exactly
 * symmetric; it also holds working data during the call, so it must not alias A.
 * eigvals: NULL or [N,B] receives w (unordered; column j of Q belongs to w_j).
 * sweeps:  NULL or [N] receives the number of sweeps run per block over both passes (each pass
 *          ends with a sweep that rotated nothing unless max_sweeps cut it short).
 * status:  NULL or [N]: bit 0 when an eigenvalue is not finite or not > 0 (X_i is NaN), bit 1 for a
 *          non-finite output, bit 2 when max_sweeps ended the last pass before it converged. */
dash_status dash_inverse_root_evd(const float* A, int64_t N, int32_t B, int32_t max_sweeps, int32_t refine, float* X,
                                  float* eigvals, int32_t* sweeps, int32_t* status, void* ws, size_t ws_bytes,
                                  void* stream);

/* dash_inverse_root_evd with the arithmetic of its first pass chosen by prec ([PT] Resultados
 * Experimentais: the eigendecomposition root, like the coupled Newton one, works with FP16 operands).
 * DASH_FP32: the same as dash_inverse_root_evd.  DASH_FP16 (refine must be 1): in the first pass every
 * product that rotates the off-pair blocks of A or the eigenvector estimate, M R with R a pair's
 * accumulated rotation, is formed as M + M (R - I), the correction from binary16 operands on the
 * binary16 matrix cores with fp32 accumulation, added to the fp32 M; A's tiles are scaled by a
 * power of two per block first (the largest diagonal entry to at most 1) and R - I is stored in
 * binary16 with a power-of-two scale per pair.  Like every first pass that a refinement pass
 * follows, it solves the 64 x 64 pair sub-problems in fp32; it leaves pairs with
 * |A_pq| <= 2^-11 sqrt(A_pp A_qq) alone (binary16's resolution).  The estimate then gets two
 * Newton-Schulz steps instead of one, and the refinement pass (fp32 products, fp64 pair
 * sub-problems, fp32 tolerance) forms H from the input again, so the result keeps fp32 accuracy.
 * A and the estimate stay fp32 in memory.  Other arguments, outputs and workspace as
 * dash_inverse_root_evd; DASH_ERR_INVALID_ARG for another prec or for DASH_FP16 with refine = 0. */
dash_status dash_inverse_root_evd_prec(const float* A, int64_t N, int32_t B, int32_t max_sweeps, int32_t refine,
                                       dash_prec prec, float* X, float* eigvals, int32_t* sweeps, int32_t* status,
                                       void* ws, size_t ws_bytes, void* stream);

/* Preconditioned update U_t = (XL_t G_t) XR_t for t < NG ([TG] body: the -1/4 powers of L and R
 * precondition the gradient).  XL, XR, G_stack, U_stack are [NG,B,B]; U_stack must not alias the
 * inputs.  ws holds one [NG,B,B] intermediate and the magnitude bounds that DASH_FP32_SPLIT16
 * uses (dash_workspace_size(DASH_OP_APPLY), the same for every prec). */
dash_status dash_apply(const float* XL, const float* XR, const float* G_stack, int64_t NG, int32_t B, float* U_stack,
                       void* ws, size_t ws_bytes, void* stream);

/* dash_apply with the products' arithmetic chosen by prec: DASH_FP32 (the fp32 matrix cores; the
 * same as dash_apply) or DASH_FP32_SPLIT (both products formed from exact three-piece bfloat16
 * splits of their fp32 operands on the bfloat16 matrix cores when B % 256 == 0; with other B the
 * fp32 matrix cores) or DASH_FP32_SPLIT16 (two-piece binary16 splits on the binary16 matrix cores,
 * each operand brought near 8 by a power of two per block: passes over XL, G and XR for their
 * bounds, and the first product's epilogue stores the intermediate's; with B % 256 != 0 the fp32
 * matrix cores).  Same workspace; DASH_ERR_INVALID_ARG for any other prec. */
dash_status dash_apply_prec(const float* XL, const float* XR, const float* G_stack, int64_t NG, int32_t B,
                            dash_prec prec, float* U_stack, void* ws, size_t ws_bytes, void* stream);

/* 1-D parameters (biases, normalisation gains).  A Shampoo preconditioner for an order-k tensor
 * takes the -1/(2k) power of each mode's statistic, so a vector (k = 1) is preconditioned by the
 * inverse square root of its one statistic; blocked like the matrices, a vector of len elements is
 * cut into ceil(len/B) pieces of B (the last zero-padded), piece p keeps L_p <- beta L_p +
 * (1 - beta) g_p g_p^T (B x B, stacked like the matrix statistics) and its update is L_p^{-1/2} g_p
 * ([TG] body: Shampoo's preconditioners come from gradient products; the pages treat weight
 * matrices only, so vectors follow Shampoo's rule for order-1 tensors).
 * dash_stack_vec: the pieces of n vectors [host descriptors] into g_pieces[P, B], vector-major, P =
 * sum ceil(len_w / B); ptr 4-byte aligned, len >= 1.  dash_unstack_vec: the first len_w elements of
 * each vector's pieces back (the padding is not written). */
dash_status dash_stack_vec(const dash_vec* grads, int32_t n, int32_t B, float* g_pieces, void* stream);
dash_status dash_unstack_vec(const float* u_pieces, int32_t B, const dash_vec* outs, int32_t n, void* stream);

/* L_p <- beta L_p + (1 - beta) g_p g_p^T for the P pieces g_pieces[P, B]; L [P, B, B] in place (each
 * block symmetric on input stays exactly symmetric).  0 <= beta <= 1. */
dash_status dash_update_stats_vec(const float* g_pieces, int64_t P, int32_t B, float beta, float* L, void* stream);

/* Inverse square root by one Newton-Denman-Beavers call ([PT] Metodologia, item 2, "Iteração de
 * Newton-Denman-Beavers": one call yields the square root and the inverse square root): iters steps
 * on A_i / s_i give Z ~ (A_i/s_i)^{-1/2}, and X_i = s_i^{-1/2} Z.  3 iters - 3 products (1 for iters
 * = 1).  prec DASH_FP32 or DASH_FP32_SPLIT (as dash_inverse_root_ndb_prec); monitor NULL or
 * [N, iters]; workspace dash_workspace_size(DASH_OP_NDB, ...).  Other arguments as
 * dash_inverse_root_ndb. */
dash_status dash_inverse_sqrt_ndb(const float* A, const float* s, int64_t N, int32_t B, int32_t iters, dash_prec prec,
                                  float* X, float* monitor, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* u_p = X_p g_p for p < P (X [P, B, B], g_pieces and u_pieces [P, B]; u must not alias g). */
dash_status dash_apply_vec(const float* X, const float* g_pieces, int64_t P, int32_t B, float* u_pieces, void* stream);

/* Workspace bytes for an operation.  k_or_degree: the number of start vectors for
 * DASH_OP_SCALE (power iteration; Frobenius needs 0), ignored otherwise.  DASH_OP_STATS: 0, or
 * with DASH_FP32_SPLIT16 the bound per tile that dash_update_stats_ws keeps (N = tiles).
 * bytes [host]. */
dash_status dash_workspace_size(dash_op op, int64_t N, int32_t B, dash_prec prec, int32_t k_or_degree,
                                size_t* bytes);

/* Number of B x B products a solver call enqueues per block (host-side count, no GPU work).
 * op: DASH_OP_NDB (iters1, iters2), DASH_OP_CN (iters1), DASH_OP_CHEB (iters1 = degree). -1 if invalid. */
int64_t dash_solver_products(dash_op op, int32_t iters1, int32_t iters2);

/* Floating-point operations one call executes on the matrix cores, counted per computed output tile
 * (host-side, no GPU work).  The Coupled-Newton, Chebyshev and statistics products compute only the
 * upper-triangle tiles of their symmetric results, so they count tdim(tdim+1)/2 of the tdim^2
 * tiles of each product (Coupled-Newton only with binary16 operands).  op and a1/a2: DASH_OP_NDB (iters1, iters2), DASH_OP_CN (iters, -),
 * DASH_OP_CHEB (degree, -), DASH_OP_APPLY (-, -; N = tiles), DASH_OP_STATS (-, -; N = tiles),
 * DASH_OP_SCALE (steps of power iteration, -), DASH_OP_EVD (sweeps, -: the products of that many
 * full sweeps plus the final X = Y Y^T).  Returns -1 for invalid arguments. */
double dash_flops(dash_op op, int64_t N, int32_t B, dash_prec prec, int32_t a1, int32_t a2);

const char* dash_status_string(dash_status status);
int32_t dash_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H_ */
