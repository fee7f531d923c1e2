// gemm_split.hip -- batched fp32 B x B products on the bfloat16 matrix cores.
//
// Each fp32 operand element x is cut into three bfloat16 pieces, x0 = bf16(x), x1 = bf16(x - x0),
// x2 = x - x0 - x1, and the cut is exact: x's 24-bit significand leaves at most 16 significant
// bits in x - x0 and at most 8 in x - x0 - x1, every difference is exact in fp32 and x2 fits
// bfloat16's 8 bits (for |x| above 2^-100, far below any operand here).  A product of two pieces
// has at most 16 significant bits, so the 32x32x16 bfloat16 MFMA forms it exactly and accumulates
// it in fp32.  The product X Y is the sum of the six piece products x_i y_j with i + j <= 2; the
// three left out are below 2^-23 of |x||y| element by element, the size of fp32's own rounding.
// The pages fix the iterations' arithmetic as fp32 and say nothing of how a matrix unit forms a
// product; this is one way to form an fp32 product, measured against fp64 to be as accurate as
// the fp32 MFMA.  On this chip the bfloat16 matrix rate is 16 times the fp32 one, so six products of
// pieces cost 6/16 of one fp32 product in MFMA time.
//
// Operands stay fp32 in memory (the same HBM bytes as the fp32 kernel); the split happens while a
// k-slice moves from the register ring to LDS, where each operand slice is held as three bfloat16
// planes.  Shape: TILE = 256 output tile, 8 waves of 128 x 64 (two per SIMD), k-slice 16 (one MFMA
// depth), a 4-deep register ring, LDS double buffer of 2 x 6 planes (96 KiB).  Both operands sit in
// LDS as rows of 16 consecutive k per output row (X) or output column (Y).
// SYM (symmetric results: Chebyshev): upper-triangle tiles, mirrored on store; the right operand
// must then be exactly symmetric (Y^T == Y bitwise, as every Clenshaw term b_{k+1} is: it is stored
// mirrored), so its columns are read as rows with 32-byte row loads; the same staging with a
// general Y forms X Y^T (the statistics' G G^T).  YT (general right operand: NDB, apply): each
// thread loads 8 consecutive k of one Y column with scalar loads (the lanes of a wave read 64
// consecutive columns, 256 contiguous bytes per load) and stores them as that column's 16-byte
// LDS row piece; XT gathers the left operand's columns the same way (X^T Y, the statistics'
// G^T G).  The epilogue reads E, and C unless FOLD: when C is Y itself (Clenshaw's b_{k+1}),
// alpha X Y + beta Y = alpha (X + (beta/alpha) I) Y, so beta/alpha is added to X's diagonal as it
// is staged (before the split) and no C is read.  (Adding C from the staged Y planes, as the fp32
// kernel does, spilled registers and measured slower.)
//
// H2 (two-piece binary16 form, Clenshaw launches): each fp32 element is first brought to binary16's
// upper range by a power of two per operand and block, x' = 2^e x with e from a bound m on |x|
// (2^13 <= 2^e m < 2^14), then cut into two binary16 pieces, x0 = f16(x') and x1 = f16(x' - x0) (the
// difference is exact in fp32), so that x' = x0 + x1 up to binary16's rounding of x1: 2^-22 |x'|,
// or 2^-25 where x1 falls below binary16's normal range, which is 2^-38 of the block's largest
// element.  x'y' = x0 y0 + x0 y1 + x1 y0 up to the term x1 y1 (2^-22 |x'||y'|): three binary16 MFMA
// products into one fp32 accumulator (piece products up to 2^28), which the epilogue multiplies by
// 2^-(ex + ey).  LDS holds two planes per operand.  The bounds: m_X = max|A| + |c| for the left
// operand A + c I (max|A| from a pass over the stack before the solve), and for the right operand
// b_{k+1} the largest of the per-wave maxima that the launch which wrote it stored in its epilogue
// (one value per wave of every tile of the block, so no atomics and no clearing).  General NN
// products (NDB's iterates, the right operand gathered by columns) take the same form, each
// operand's bound the per-wave maxima of the launch that wrote it, or a pass over it.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gemm_common.hpp"

namespace dash {
namespace gemm {
namespace {

template <int V>
using IC = std::integral_constant<int, V>;

// x = p0 + p1 + p2 for the 8 elements lo[0..3], hi[0..3]
__device__ __forceinline__ void split3(const f32x4& lo, const f32x4& hi, bf16x8& p0, bf16x8& p1, bf16x8& p2) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float x = q < 4 ? lo[q] : hi[q - 4];
    const __bf16 a0 = (__bf16)x;
    const float r1 = x - (float)a0;
    const __bf16 a1 = (__bf16)r1;
    p0[q] = a0;
    p1[q] = a1;
    p2[q] = (__bf16)(r1 - (float)a1);
  }
}

// power-of-two exponent e with 2^13 <= 2^e m < 2^14 (m = 0, inf or NaN: 0)
__device__ __forceinline__ int top_exp(float m) {
  int e;
  frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)
  return (m > 0.f && isfinite(m)) ? 14 - e : 0;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// H2 pieces of the 8 elements lo[0..3], hi[0..3] of 2^e x: x0 = f16(x'), x1 = f16(x' - x0).  The
// difference is formed by one mixed-precision fma of x0 (binary16 source) with -1; m1 holds -1 where
// the compiler cannot see it, so that it keeps the fma instead of a conversion and a subtraction.
__device__ __forceinline__ void split2(const f32x4& lo, const f32x4& hi, int e, float m1, f16x8& p0, f16x8& p1) {
#pragma unroll
  for (int q = 0; q < 8; q += 2) {
    const float a = ldexpf(q < 4 ? lo[q] : hi[q - 4], e);
    const float b = ldexpf(q < 4 ? lo[q + 1] : hi[q - 3], e);
    const f16x2 h = __builtin_convertvector(f32x2{a, b}, f16x2);
    const f32x2 r = {__builtin_fmaf((float)h[0], m1, a), __builtin_fmaf((float)h[1], m1, b)};
    const f16x2 l = __builtin_convertvector(r, f16x2);
    p0[q] = h[0];
    p0[q + 1] = h[1];
    p1[q] = l[0];
    p1[q + 1] = l[1];
  }
}

// LDS rows are 16 bfloat16 (two 16-byte chunks); a row swaps its chunks when bit 2 xor bit 3 of its
// index is set, so that the 16-byte reads of 16 consecutive rows (one chunk each, the lanes the LDS
// serves together) fall on 16 distinct 16-byte slots of its 64 banks
__device__ __forceinline__ int swz2(int row, int ch) { return ch ^ ((row >> 2) & 1) ^ ((row >> 3) & 1); }

template <bool CHECKS, bool SYM, bool XT, bool YT, bool FOLD = false, bool H2 = false>
__global__ __launch_bounds__(512) void gemm_split_kernel(GemmArgs a) {
  constexpr int TILE = 256, BK = 16, DEPTH = 4;
  constexpr int WTM = 128, WTN = 64, MTM = 4, MTN = 2;
  using TE = std::conditional_t<H2, _Float16, __bf16>;
  using V8 = typename Half<TE>::v8;
  constexpr int PLANE = TILE * BK;           // elements of one piece plane of one operand slice
  constexpr int YP = H2 ? 2 : 3;             // pieces per operand
  constexpr int BUF = 2 * YP * PLANE;        // X pieces, then Y pieces
  // the two stages of the double buffer are separate arrays: the stores of one stage and the
  // reads of the other then provably do not alias, so the compiler may interleave the staging of
  // slice k + 1 (split and LDS stores) with the products of slice k
  __shared__ __attribute__((aligned(16))) TE stage0[BUF];
  __shared__ __attribute__((aligned(16))) TE stage1[BUF];
  auto smem_of = [&](int buf) -> TE* { return buf ? stage1 : stage0; };

  const TileCoord tc = decode_tile(a, SYM);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const float* X = (const float*)P.X + off;
  const float* Y = (const float*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int wm = wave >> 2, wn = wave & 3;
  // H2, symmetric results: a diagonal tile keeps 36 of its 64 32 x 32 sub-blocks.  There the waves
  // take the 128 x 64 regions so that the two waves of each SIMD (waves w and w + 4) hold at most 11
  // kept sub-blocks, and the products of the others are skipped (their values are never stored)
  unsigned need = 0xffu;
  if (H2 && SYM && tc.ti == tc.tj) {
    const int w = __builtin_amdgcn_readfirstlane(wave);
    wm = (0xD8 >> w) & 1;          // regions (0,2) (0,3) (0,1) (1,3) (1,2) (0,0) (1,0) (1,1)
    wn = (17118 >> (2 * w)) & 3;
    need = 0;
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
        if (wm * WTM + mt * 32 <= wn * WTN + nt * 32) need |= 1u << (mt * MTN + nt);
    need = __builtin_amdgcn_readfirstlane(need);
  }
  const int li = lane & 31, h = lane >> 5;
  const int srow = tid >> 1, sch = tid & 1;    // row piece: row srow, k 8 sch .. 8 sch + 7
  const int gcol = tid & 255, gkh = tid >> 8;  // column gather: column gcol, k 8 gkh .. 8 gkh + 7
  const int xrow = XT ? gcol : srow, xch = XT ? gkh : sch;  // the pieces' LDS rows and chunks
  const int yrow = YT ? gcol : srow, ych = YT ? gkh : sch;

  // Column gathers read the operand's block as a buffer (out-of-range reads return 0; every
  // offset here is in range): the row offset is wave-uniform (a scalar), the lane's column and
  // k-half a 32-bit byte offset.  The block's address is the same in every lane; say so, or every
  // load becomes a loop over the distinct descriptors of the wave.
  auto block_rsrc = [&](const float* p) {
    const uint64_t a64 = (uint64_t)p;
    const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a64 >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a64);
    return __builtin_amdgcn_make_buffer_rsrc((void*)u, (short)0, B * B * 4, BUFFER_RSRC_WORD3);
  };
  __amdgpu_buffer_rsrc_t xrs, yrs;
  int xvoff = 0, yvoff = 0;
  if constexpr (XT) {
    xrs = block_rsrc(X);
    xvoff = (8 * gkh * B + i0 + gcol) * 4;
  }
  if constexpr (YT) {
    yrs = block_rsrc(Y);
    yvoff = (8 * gkh * B + j0 + gcol) * 4;
  }

  f32x4 rx[DEPTH][2], ry[DEPTH][2];
  auto gather = [&](f32x4 (&r)[2], __amdgpu_buffer_rsrc_t rs, int voff, int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q)  // (the load returns the word's bits as an integer)
      r[q >> 2][q & 3] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, (k0 + q) * B * 4, 0));
  };
  auto gload = [&](auto slot_c, int k0) {
    constexpr int slot = decltype(slot_c)::value;
    if constexpr (XT) {
      gather(rx[slot], xrs, xvoff, k0);
    } else {
      const float* xp = X + (int64_t)(i0 + srow) * B + k0 + 8 * sch;
      rx[slot][0] = *(const f32x4*)xp;
      rx[slot][1] = *(const f32x4*)(xp + 4);
    }
    if constexpr (YT) {
      gather(ry[slot], yrs, yvoff, k0);
    } else {
      const float* yp = Y + (int64_t)(j0 + srow) * B + k0 + 8 * sch;
      ry[slot][0] = *(const f32x4*)yp;
      ry[slot][1] = *(const f32x4*)(yp + 4);
    }
  };
  // FOLD (C == Y, Clenshaw's b_{k+1}): alpha X Y + beta Y = alpha (X + (beta/alpha) I) Y, so the
  // C term enters as (beta/alpha) added to X's diagonal before the split, and no C is read
  const float xc = FOLD ? a.epi.c_over_a * coef_of(a.epi, a.epi.ic, tc.b) : 0.f;
  // H2: the operands' power-of-two exponents for this block (every wave reduces the right
  // operand's per-wave maxima itself)
  int ex = 0, ey = 0;
  float m1 = -1.f;
  if constexpr (H2) {
    const float* xb = P.amax_x + tc.b * P.amax_x_parts;
    const float* yb = P.amax_y + tc.b * P.amax_y_parts;
    float mx = 0.f, my = 0.f;
    for (int p = lane; p < P.amax_x_parts; p += 64) mx = fmaxf(mx, xb[p]);
    for (int p = lane; p < P.amax_y_parts; p += 64) my = fmaxf(my, yb[p]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      my = fmaxf(my, __shfl_xor(my, o, 64));
    }
    // (the same in every lane: keep them scalar)
    ex = __builtin_amdgcn_readfirstlane(top_exp(mx + fabsf(xc)));
    ey = __builtin_amdgcn_readfirstlane(top_exp(my));
    asm("" : "+s"(m1));  // (no instruction: hides the constant -1 from the optimiser)
  }
  auto sstore = [&](auto slot_c, int buf, int k0) {
    constexpr int slot = decltype(slot_c)::value;
    TE* s = smem_of(buf) + xrow * BK + 8 * swz2(xrow, xch);
    // element q of the piece sits on the diagonal when i0 + row == k0 + 8 ch + q: only the slices
    // with k0 in (i0 - BK, i0 + TILE) hold diagonal elements of the tile's rows.  H2 skips the others
    // by a uniform branch (the bfloat16 form measured faster without it)
    if (FOLD && (!H2 || (k0 + BK > i0 && k0 < i0 + TILE))) {
      const int d = i0 + srow - k0 - 8 * sch;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rx[slot][0][q] = d == q ? rx[slot][0][q] + xc : rx[slot][0][q];
        rx[slot][1][q] = d == q + 4 ? rx[slot][1][q] + xc : rx[slot][1][q];
      }
    }
    TE* t = smem_of(buf) + YP * PLANE + yrow * BK + 8 * swz2(yrow, ych);
    if constexpr (H2) {
      f16x8 p0, p1;
      split2(rx[slot][0], rx[slot][1], ex, m1, p0, p1);
      *(f16x8*)(s) = p0;
      *(f16x8*)(s + PLANE) = p1;
      split2(ry[slot][0], ry[slot][1], ey, m1, p0, p1);
      *(f16x8*)(t) = p0;
      *(f16x8*)(t + PLANE) = p1;
    } else {
      bf16x8 p0, p1, p2;
      split3(rx[slot][0], rx[slot][1], p0, p1, p2);
      *(bf16x8*)(s) = p0;
      *(bf16x8*)(s + PLANE) = p1;
      *(bf16x8*)(s + 2 * PLANE) = p2;
      split3(ry[slot][0], ry[slot][1], p0, p1, p2);
      *(bf16x8*)(t) = p0;
      *(bf16x8*)(t + PLANE) = p1;
      *(bf16x8*)(t + 2 * PLANE) = p2;
    }
  };

  f32x16 acc[MTM][MTN];
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  // one k-slice: lane half h takes k = 8h .. 8h + 7 of the slice for both operands.  H2: both
  // right pieces and both left pieces of the wave's fragments, then x0 y0, x0 y1 and x1 y0.
  auto compute_h2 = [&](int buf) {
    const TE* s = smem_of(buf);
    auto frag = [&](int plane, int row) { return *(const V8*)&s[plane * PLANE + row * BK + 8 * swz2(row, h)]; };
    V8 y0[MTN], y1[MTN], x0[MTM], x1[MTM];
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt) y0[nt] = frag(2, wn * WTN + nt * 32 + li);
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt) x0[mt] = frag(0, wm * WTM + mt * 32 + li);
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt) y1[nt] = frag(3, wn * WTN + nt * 32 + li);
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt) x1[mt] = frag(1, wm * WTM + mt * 32 + li);
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
        if ((need >> (mt * MTN + nt)) & 1) acc[mt][nt] = Half<TE>::mfma(x0[mt], y0[nt], acc[mt][nt]);
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
        if ((need >> (mt * MTN + nt)) & 1) acc[mt][nt] = Half<TE>::mfma(x0[mt], y1[nt], acc[mt][nt]);
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
        if ((need >> (mt * MTN + nt)) & 1) acc[mt][nt] = Half<TE>::mfma(x1[mt], y0[nt], acc[mt][nt]);
  };
  // bfloat16: one right piece at a time (its two fragments), each left piece read per use
  auto compute = [&](int buf) {
    if constexpr (H2) {
      compute_h2(buf);
      return;
    }
    const TE* s = smem_of(buf);
#pragma unroll
    for (int pb = 0; pb < 3; ++pb) {
      V8 bv[MTN];
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt) {
        const int row = wn * WTN + nt * 32 + li;
        bv[nt] = *(const V8*)&s[(3 + pb) * PLANE + row * BK + 8 * swz2(row, h)];
      }
#pragma unroll
      for (int pa = 0; pa + pb < 3; ++pa)
#pragma unroll
        for (int mt = 0; mt < MTM; ++mt) {
          const int row = wm * WTM + mt * 32 + li;
          const V8 av = *(const V8*)&s[pa * PLANE + row * BK + 8 * swz2(row, h)];
#pragma unroll
          for (int nt = 0; nt < MTN; ++nt) acc[mt][nt] = Half<TE>::mfma(av, bv[nt], acc[mt][nt]);
        }
    }
  };

  const int KT = B / BK;  // a multiple of 16 (B % 256 == 0)
  // Steady state: the loads of slice kt + DEPTH go into the registers slice kt vacated, slice
  // kt + 1 moves from registers to the other LDS buffer, then the MFMAs consume slice kt.
  auto step = [&](auto slot_c, int kt) {
    constexpr int slot = decltype(slot_c)::value;  // == kt % DEPTH
    gload(slot_c, (kt + DEPTH) * BK);
    sstore(IC<(slot + 1) % DEPTH>{}, (slot + 1) & 1, (kt + 1) * BK);
    compute(slot & 1);
    __syncthreads();
  };
  auto tail_step = [&](auto slot_c, int kt, bool store_next) {
    constexpr int slot = decltype(slot_c)::value;
    if (store_next) sstore(IC<(slot + 1) % DEPTH>{}, (slot + 1) & 1, (kt + 1) * BK);
    compute(slot & 1);
    __syncthreads();
  };
  gload(IC<0>{}, 0);
  gload(IC<1>{}, BK);
  gload(IC<2>{}, 2 * BK);
  gload(IC<3>{}, 3 * BK);
  sstore(IC<0>{}, 0, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + DEPTH < KT; kt += DEPTH) {
    step(IC<0>{}, kt);
    step(IC<1>{}, kt + 1);
    step(IC<2>{}, kt + 2);
    step(IC<3>{}, kt + 3);
  }
  tail_step(IC<0>{}, kt, true);
  tail_step(IC<1>{}, kt + 1, true);
  tail_step(IC<2>{}, kt + 2, true);
  tail_step(IC<3>{}, kt + 3, false);
  if constexpr (H2) {
    const int es = -ex - ey;
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][nt][r] = ldexpf(acc[mt][nt][r], es);
  }
  // H2: this wave's slot among the block's per-wave maxima (tile index t, 8 waves; symmetric
  // results number the upper-triangle tiles row by row)
  float* amax_out = nullptr;
  if (H2 && P.amax_d) {
    const int t = SYM ? tc.ti * a.tdim - tc.ti * (tc.ti - 1) / 2 + (tc.tj - tc.ti) : tc.ti * a.tdim + tc.tj;
    amax_out = P.amax_d + (tc.b * a.tiles + t) * 8 + wave;
  }
  // symmetric results mirror through LDS (the stage buffers are free after the loop's last barrier)
  static_assert(!SYM || 8 * MLDS_FLOATS * sizeof(float) <= 2 * BUF * sizeof(TE), "LDS for the mirror");
  float* mlds = SYM ? (float*)(wave < 4 ? (void*)stage0 : (void*)stage1) + (wave & 3) * MLDS_FLOATS : nullptr;
  epilogue_split<MTM, MTN, WTM, WTN, SYM, !FOLD, TILE, CHECKS, H2>(a, tc, P, acc, wm, wn, lane, amax_out, mlds);
}

}  // namespace

hipError_t launch_split(GemmArgs& a, bool sym, Trans trans, bool y_sym, bool h2, hipStream_t stream) {
  if (a.B % 256 != 0) return hipErrorInvalidValue;
  a.tdim = a.B / 256;
  a.tiles = sym ? a.tdim * (a.tdim + 1) / 2 : a.tdim * a.tdim;
  const bool checks = wants_checks(a.epi);
  // two-piece binary16 form: the Clenshaw launches (symmetric NN with C == Y folded), general NN
  // products (NDB's iterates, the apply) and the statistics' symmetric G G^T (NT) and G^T G (TN)
  if (h2) {
    if (trans != Trans::NN) {
      if (!sym || a.epi.fold_c) return hipErrorInvalidValue;
      if (trans == Trans::NT)
        return checks ? launch(gemm_split_kernel<true, true, false, false, false, true>, a, stream, 512)
                      : launch(gemm_split_kernel<false, true, false, false, false, true>, a, stream, 512);
      return checks ? launch(gemm_split_kernel<true, true, true, true, false, true>, a, stream, 512)
                    : launch(gemm_split_kernel<false, true, true, true, false, true>, a, stream, 512);
    }
    if (sym != a.epi.fold_c) return hipErrorInvalidValue;
    if (!sym)
      return checks ? launch(gemm_split_kernel<true, false, false, true, false, true>, a, stream, 512)
                    : launch(gemm_split_kernel<false, false, false, true, false, true>, a, stream, 512);
    if (y_sym)
      return checks ? launch(gemm_split_kernel<true, true, false, false, true, true>, a, stream, 512)
                    : launch(gemm_split_kernel<false, true, false, false, true, true>, a, stream, 512);
    return checks ? launch(gemm_split_kernel<true, true, false, true, true, true>, a, stream, 512)
                  : launch(gemm_split_kernel<false, true, false, true, true, true>, a, stream, 512);
  }
  // symmetric results: NN of an exactly symmetric Y and NT read Y's rows as B's columns; TN
  // gathers the columns of both operands; NN with C == Y folded gathers Y's columns unless Y is
  // exactly symmetric.  General results: NN with Y's columns gathered.
  if (sym && trans == Trans::NN && a.epi.fold_c) {  // C == Y folded into X's diagonal
    if (y_sym)
      return checks ? launch(gemm_split_kernel<true, true, false, false, true>, a, stream, 512)
                    : launch(gemm_split_kernel<false, true, false, false, true>, a, stream, 512);
    return checks ? launch(gemm_split_kernel<true, true, false, true, true>, a, stream, 512)
                  : launch(gemm_split_kernel<false, true, false, true, true>, a, stream, 512);
  }
  if (a.epi.fold_c) return hipErrorInvalidValue;
  if (sym && (trans == Trans::NT || (trans == Trans::NN && y_sym)))
    return checks ? launch(gemm_split_kernel<true, true, false, false>, a, stream, 512)
                  : launch(gemm_split_kernel<false, true, false, false>, a, stream, 512);
  if (sym && trans == Trans::TN)
    return checks ? launch(gemm_split_kernel<true, true, true, true>, a, stream, 512)
                  : launch(gemm_split_kernel<false, true, true, true>, a, stream, 512);
  if (!sym && trans == Trans::NN)
    return checks ? launch(gemm_split_kernel<true, false, false, true>, a, stream, 512)
                  : launch(gemm_split_kernel<false, false, false, true>, a, stream, 512);
  return hipErrorInvalidValue;
}

}  // namespace gemm
}  // namespace dash
