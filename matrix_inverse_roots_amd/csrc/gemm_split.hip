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

// Word 3 of a raw buffer resource on this architecture: 32-bit data format, no swizzle, byte
// offsets (the loads here are untyped).
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

// LDS rows are 16 bfloat16 (two 16-byte chunks); a row swaps its chunks when bit 2 xor bit 3 of its
// index is set, so that the 16-byte reads of 16 consecutive rows (one chunk each, the lanes the LDS
// serves together) fall on 16 distinct 16-byte slots of its 64 banks
__device__ __forceinline__ int swz2(int row, int ch) { return ch ^ ((row >> 2) & 1) ^ ((row >> 3) & 1); }

template <bool CHECKS, bool SYM, bool XT, bool YT, bool FOLD = false>
__global__ __launch_bounds__(512) void gemm_split_kernel(GemmArgs a) {
  constexpr int TILE = 256, BK = 16, DEPTH = 4;
  constexpr int WTM = 128, WTN = 64, MTM = 4, MTN = 2;
  constexpr int PLANE = TILE * BK;  // bfloat16 of one piece plane of one operand slice
  constexpr int BUF = 6 * PLANE;    // X pieces 0..2, then Y pieces 0..2
  // the two stages of the double buffer are separate arrays: the stores of one stage and the
  // reads of the other then provably do not alias, so the compiler may interleave the staging of
  // slice k + 1 (split and LDS stores) with the products of slice k
  __shared__ __attribute__((aligned(16))) __bf16 stage0[BUF];
  __shared__ __attribute__((aligned(16))) __bf16 stage1[BUF];
  auto smem_of = [&](int buf) -> __bf16* { return buf ? stage1 : stage0; };

  const TileCoord tc = decode_tile(a, SYM);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const float* X = (const float*)P.X + off;
  const float* Y = (const float*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
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
  auto sstore = [&](auto slot_c, int buf, int k0) {
    constexpr int slot = decltype(slot_c)::value;
    __bf16* s = smem_of(buf) + xrow * BK + 8 * swz2(xrow, xch);
    bf16x8 p0, p1, p2;
    if constexpr (FOLD) {  // element q of the piece sits on the diagonal when i0 + row == k0 + 8 ch + q
      const int d = i0 + srow - k0 - 8 * sch;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rx[slot][0][q] = d == q ? rx[slot][0][q] + xc : rx[slot][0][q];
        rx[slot][1][q] = d == q + 4 ? rx[slot][1][q] + xc : rx[slot][1][q];
      }
    }
    split3(rx[slot][0], rx[slot][1], p0, p1, p2);
    *(bf16x8*)(s) = p0;
    *(bf16x8*)(s + PLANE) = p1;
    *(bf16x8*)(s + 2 * PLANE) = p2;
    __bf16* t = smem_of(buf) + 3 * PLANE + yrow * BK + 8 * swz2(yrow, ych);
    split3(ry[slot][0], ry[slot][1], p0, p1, p2);
    *(bf16x8*)(t) = p0;
    *(bf16x8*)(t + PLANE) = p1;
    *(bf16x8*)(t + 2 * PLANE) = p2;
  };

  f32x16 acc[MTM][MTN];
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  // one k-slice: lane half h takes k = 8h .. 8h + 7 of the slice for both operands; one right
  // piece at a time (its two fragments), each left piece read per use
  auto compute = [&](int buf) {
    const __bf16* s = smem_of(buf);
#pragma unroll
    for (int pb = 0; pb < 3; ++pb) {
      bf16x8 bv[MTN];
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt) {
        const int row = wn * WTN + nt * 32 + li;
        bv[nt] = *(const bf16x8*)&s[(3 + pb) * PLANE + row * BK + 8 * swz2(row, h)];
      }
#pragma unroll
      for (int pa = 0; pa + pb < 3; ++pa)
#pragma unroll
        for (int mt = 0; mt < MTM; ++mt) {
          const int row = wm * WTM + mt * 32 + li;
          const bf16x8 av = *(const bf16x8*)&s[pa * PLANE + row * BK + 8 * swz2(row, h)];
#pragma unroll
          for (int nt = 0; nt < MTN; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[nt], acc[mt][nt], 0, 0, 0);
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
  epilogue<MTM, MTN, WTM, WTN, SYM, float, !FOLD, true, TILE, CHECKS, false, false>(a, tc, P, acc, wm, wn, lane);
}

}  // namespace

hipError_t launch_split(GemmArgs& a, bool sym, Trans trans, bool y_sym, hipStream_t stream) {
  if (a.B % 256 != 0) return hipErrorInvalidValue;
  a.tdim = a.B / 256;
  a.tiles = sym ? a.tdim * (a.tdim + 1) / 2 : a.tdim * a.tdim;
  const bool checks = wants_checks(a.epi);
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
