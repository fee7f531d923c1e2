// gemm_f16.hip -- batched B x B products with 2-byte operands (binary16 or bfloat16, the element
// type TE) and fp32 accumulation on the 32x32x16 MFMA (the half-precision solvers).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gemm_common.hpp"

namespace dash {
namespace gemm {
namespace {

template <typename TE, int TILE, bool SYM, typename TO, bool CHECKS, bool FRZ = false>
__global__ __launch_bounds__(256) void gemm_f16_kernel(GemmArgs a) {
  typedef typename Half<TE>::v8 V8;
  constexpr int BK = 64;
  constexpr int WT = TILE / 2;
  constexpr int MT = WT / 32;
  constexpr int LD = BK + 8;  // As[m][k], Bs[n][k] (Y tile transposed)
  constexpr int NL = TILE * BK / 8 / 256;
  constexpr int SMEM_BYTES = 2 * 2 * TILE * LD * 2;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  TE(*As)[TILE * LD] = reinterpret_cast<TE(*)[TILE * LD]>(smem);
  TE(*Bs)[TILE * LD] = reinterpret_cast<TE(*)[TILE * LD]>(smem + 2 * TILE * LD * 2);

  TileCoord tc;
  if constexpr (FRZ) {
    if (!decode_tile_interleaved(a, SYM, tc)) return;
  } else {
    tc = decode_tile(a, SYM);
  }
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const TE* X = (const TE*)P.X + off;
  const TE* Y = (const TE*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  if constexpr (FRZ) {  // a block that stopped iterating: pass an operand through, or write nothing
    if (P.freeze && P.freeze[tc.b]) {
      if (P.pass == 0) return;
      f32x16 pz[MT][MT];
      pass_tile_f16<TE, MT, MT, WT, WT>(P, X, Y, B, i0, j0, wm, wn, lane, pz);
      if constexpr (sizeof(TO) == 2)
        epilogue_staged_f16<TE, MT, MT, WT, WT, SYM, TILE, CHECKS>(a, tc, P, pz, wm, wn, lane, smem);
      else
        epilogue<MT, MT, WT, WT, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, pz, wm, wn, lane);
      return;
    }
  }

  V8 ra[NL], rb[NL];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      ra[r] = *(const V8*)(X + (int64_t)(i0 + row) * B + k0 + 8 * c8);
      const int krow = f / (TILE / 8), n8 = f % (TILE / 8);
      rb[r] = *(const V8*)(Y + (int64_t)(k0 + krow) * B + j0 + 8 * n8);
    }
  };
  auto sstore = [&](int buf, int k0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      const int krow = f / (TILE / 8), n8 = f % (TILE / 8);
      const V8 xa = P.map_x ? operand_map<TE>(ra[r], i0 + row, k0 + 8 * c8, P.map_a, P.map_g) : ra[r];
      const V8 yb = P.map_y ? operand_map<TE>(rb[r], k0 + krow, j0 + 8 * n8, P.map_a, P.map_g) : rb[r];
      *(V8*)&As[buf][row * LD + 8 * c8] = xa;
#pragma unroll
      for (int q = 0; q < 8; ++q) Bs[buf][(8 * n8 + q) * LD + krow] = yb[q];
    }
  };

  f32x16 acc[MT][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < MT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  const int KT = B / BK;
  gload(0);
  sstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const TE* as = As[buf];
    const TE* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      V8 av[MT], bv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = *(const V8*)&as[(wm * WT + mt * 32 + li) * LD + h * 32 + 8 * s];
#pragma unroll
      for (int nt = 0; nt < MT; ++nt) bv[nt] = *(const V8*)&bs[(wn * WT + nt * 32 + li) * LD + h * 32 + 8 * s];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < MT; ++nt)
          acc[mt][nt] = Half<TE>::mfma(av[mt], bv[nt], acc[mt][nt]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1, (kt + 1) * BK);
    __syncthreads();
  }
  if constexpr (sizeof(TO) == 2)
    epilogue_staged_f16<TE, MT, MT, WT, WT, SYM, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane, smem);
  else
    epilogue<MT, MT, WT, WT, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane);
}


// ------------------------------------------------------------------------------------------------
// fp16 operands with a general right operand (NDB with binary16 iterates), 256 x 256 macro tile
// (B % 256 == 0), no operand maps.  Four waves as 2 x 2, wave tile 128 x 128
// (4 x 4 accumulators of 32 x 32, held in the accumulation registers at one wave per SIMD).  Every
// thread stages 8 pieces of the X slice (256 rows x 64 k, 16-byte loads) and one 8 (k) x 8 (n)
// sub-block of the Y slice, loaded as eight 16-byte row pieces and transposed in registers, so both
// LDS tiles hold rows of 64 consecutive k.  LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
// (row ^ row/8) & 7, which keeps both the MFMA reads (8 consecutive rows, one chunk) and the
// transposed writes (rows 8 apart, one chunk) free of bank conflicts.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row ^ (row >> 3))) & 7; }

template <typename TE, bool SYM, typename TO, bool CHECKS>
__global__ __launch_bounds__(256) void gemm_f16_big_kernel(GemmArgs a) {
  typedef typename Half<TE>::v8 V8;
  constexpr int TILE = 256, BK = 64, MT = 4, WT = 128;
  // double-buffered X and Y slices (128 KiB); a little more so a mirrored binary16 tile fits whole
  constexpr int MAIN_BYTES = 2 * 2 * TILE * BK * 2;
  constexpr int STAGE_BYTES = TILE * (TILE + 8) * 2;  // binary16 output tile staged for 16-byte stores
  constexpr int SMEM_BYTES = MAIN_BYTES > STAGE_BYTES ? MAIN_BYTES : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  TE(*As)[TILE * BK] = reinterpret_cast<TE(*)[TILE * BK]>(smem);
  TE(*Bs)[TILE * BK] = reinterpret_cast<TE(*)[TILE * BK]>(smem + 2 * TILE * BK * 2);

  const TileCoord tc = decode_tile(a, SYM);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const TE* X = (const TE*)P.X + off;
  const TE* Y = (const TE*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;
  const int kb = tid >> 5, nb = tid & 31;  // this thread's 8 x 8 sub-block of the Y slice

  // X slice: 8 pieces of 16 bytes, piece c = tid + 256 r -> row c / 8, chunk c % 8.
  // Y slice: k rows 8 kb .. 8 kb + 7, n columns 8 nb .. 8 nb + 7, transposed in registers.
  V8 lx[8], ly[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = tid + 256 * r;
      lx[r] = *(const V8*)(X + (int64_t)(i0 + (c >> 3)) * B + k0 + 8 * (c & 7));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ly[q] = *(const V8*)(Y + (int64_t)(k0 + 8 * kb + q) * B + j0 + 8 * nb);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = tid + 256 * r;
      const int row = c >> 3;
      *(V8*)&As[buf][row * BK + 8 * swz(row, c & 7)] = lx[r];
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      V8 col;
#pragma unroll
      for (int q = 0; q < 8; ++q) col[q] = ly[q][n];
      const int row = 8 * nb + n;
      *(V8*)&Bs[buf][row * BK + 8 * swz(row, kb)] = col;
    }
  };

  f32x16 acc[MT][MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < MT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  const int KT = B / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const TE* as = As[buf];
    const TE* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 4 * h + s;
      V8 av[MT], bv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * WT + mt * 32 + li;
        av[mt] = *(const V8*)&as[row * BK + 8 * swz(row, chunk)];
      }
#pragma unroll
      for (int nt = 0; nt < MT; ++nt) {
        const int row = wn * WT + nt * 32 + li;
        bv[nt] = *(const V8*)&bs[row * BK + 8 * swz(row, chunk)];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < MT; ++nt)
          acc[mt][nt] = Half<TE>::mfma(av[mt], bv[nt], acc[mt][nt]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  if constexpr (sizeof(TO) == 2)
    epilogue_staged_f16<TE, MT, MT, WT, WT, SYM, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane, smem);
  else
    epilogue<MT, MT, WT, WT, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane);
}

// ------------------------------------------------------------------------------------------------
// fp16 operands with an exactly symmetric right operand Y (Y^T = Y bitwise), 256 x 256 macro tile,
// four waves of 128 x 128 or eight waves of 128 x 64.
// Then column j of Y is row j of Y, so both slices are read as rows of consecutive k with 16-byte
// loads and no transposition.  The k-step is 32 and the global slices run DEPTH = 4 k-steps ahead
// of the MFMAs through a ring of registers (two LDS buffers), so each workgroup keeps 128 KiB of
// loads in flight: the products of the coupled-Newton iteration are latency-bound otherwise (one
// workgroup per CU, and the first touch of every operand panel misses L2).
// LDS rows are 64 bytes; the 16-byte chunk index is XOR-swizzled by bits 2-3 of the row.  The LDS
// serves a 16-byte access 16 lanes at a time from 64 banks (256 bytes): the MFMA reads (16
// consecutive rows, one chunk) then fall on 16 distinct 16-byte slots, and so do the stores (4
// rows x 4 chunks).  (Swizzled by row/2, rows r and r + 8 shared a slot: 2-way conflicts on every
// fragment read.)
// ------------------------------------------------------------------------------------------------
template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ int swz4(int row, int chunk) { return (chunk ^ (row >> 2)) & 3; }

template <typename TE, bool SYM, typename TO, bool CHECKS, int NW, bool FRZ = false>
__global__ __launch_bounds__(64 * NW) void gemm_f16_ysym_kernel(GemmArgs a) {
  typedef typename Half<TE>::v8 V8;
  // NW = 4: 2 x 2 waves of 128 x 128; NW = 8: 2 x 4 waves of 128 x 64 (two waves per SIMD)
  constexpr int NT = 64 * NW;
  constexpr int TILE = 256, BK = 32, DEPTH = 4;
  constexpr int WTM = 128, WTN = TILE / (NW / 2), MTM = WTM / 32, MTN = WTN / 32;
  constexpr int NP = TILE * BK / 8 / NT;  // 16-byte pieces per thread per operand slice
  constexpr int SLICE = TILE * BK;  // halves of one operand slice
  constexpr int MAIN_BYTES = 2 * 2 * SLICE * 2;
  constexpr int STAGE_BYTES = TILE * (TILE + 8) * 2;  // binary16 output tile staged for 16-byte stores
  constexpr int SMEM_BYTES = MAIN_BYTES > STAGE_BYTES ? MAIN_BYTES : STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  TE* Xs = (TE*)smem;  // [2][SLICE]
  TE* Ys = Xs + 2 * SLICE;   // [2][SLICE]

  TileCoord tc;
  if constexpr (FRZ) {
    if (!decode_tile_interleaved(a, SYM, tc)) return;
  } else {
    tc = decode_tile(a, SYM);
  }
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const TE* X = (const TE*)P.X + off;
  const TE* Y = (const TE*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
  const int li = lane & 31, h = lane >> 5;

  if constexpr (FRZ) {  // a block that stopped iterating: pass an operand through, or write nothing
    if (P.freeze && P.freeze[tc.b]) {
      if (P.pass == 0) return;
      f32x16 pz[MTM][MTN];
      pass_tile_f16<TE, MTM, MTN, WTM, WTN>(P, X, Y, B, i0, j0, wm, wn, lane, pz);
      if constexpr (sizeof(TO) == 2)
        epilogue_staged_f16<TE, MTM, MTN, WTM, WTN, SYM, TILE, CHECKS>(a, tc, P, pz, wm, wn, lane, smem);
      else
        epilogue<MTM, MTN, WTM, WTN, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, pz, wm, wn, lane);
      return;
    }
  }

  // per k-step each thread moves NP pieces of 16 bytes of each slice: piece c = tid + NT r -> row
  // c / 4, chunk c % 4 (rows i0.. of X and rows j0.. of Y, k0 .. k0 + 31)
  V8 rx[DEPTH][NP], ry[DEPTH][NP];
  auto gload = [&](auto slot_c, int k0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int c = tid + NT * r;
      const int row = c >> 2, ch = c & 3;
      rx[slot][r] = *(const V8*)(X + (int64_t)(i0 + row) * B + k0 + 8 * ch);
      ry[slot][r] = *(const V8*)(Y + (int64_t)(j0 + row) * B + k0 + 8 * ch);
    }
  };
  auto sstore = [&](auto slot_c, int buf, int k0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int c = tid + NT * r;
      const int row = c >> 2, ch = c & 3;
      const int o = buf * SLICE + row * BK + 8 * swz4(row, ch);
      *(V8*)&Xs[o] = P.map_x ? operand_map<TE>(rx[slot][r], i0 + row, k0 + 8 * ch, P.map_a, P.map_g) : rx[slot][r];
      *(V8*)&Ys[o] = P.map_y ? operand_map<TE>(ry[slot][r], j0 + row, k0 + 8 * ch, P.map_a, P.map_g) : ry[slot][r];
    }
  };

  f32x16 acc[MTM][MTN];
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  auto compute = [&](int buf) {
    const TE* xs = Xs + buf * SLICE;
    const TE* ys = Ys + buf * SLICE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int chunk = 2 * h + s;
      V8 av[MTM], bv[MTN];
#pragma unroll
      for (int mt = 0; mt < MTM; ++mt) {
        const int row = wm * WTM + mt * 32 + li;
        av[mt] = *(const V8*)&xs[row * BK + 8 * swz4(row, chunk)];
      }
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt) {
        const int row = wn * WTN + nt * 32 + li;
        bv[nt] = *(const V8*)&ys[row * BK + 8 * swz4(row, chunk)];
      }
#pragma unroll
      for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
        for (int nt = 0; nt < MTN; ++nt)
          acc[mt][nt] = Half<TE>::mfma(av[mt], bv[nt], acc[mt][nt]);
    }
  };

  const int KT = B / BK;  // a multiple of 8 (B % 256 == 0)
  // Steady state: the loads of k-step kt + DEPTH go into the registers that k-step kt vacated, the
  // MFMAs consume kt from LDS, then k-step kt + 1 moves from registers to the other LDS buffer.
  // The loads are unconditional here (the tail below has none), so the compiler's wait before the
  // LDS store counts only k-step kt + 1's loads and leaves the later ones in flight.
  auto step = [&](auto slot_c, int kt) {
    constexpr int slot = decltype(slot_c)::value;  // == kt % DEPTH
    gload(slot_c, (kt + DEPTH) * BK);
    compute(slot & 1);
    sstore(IC<(slot + 1) % DEPTH>{}, (slot + 1) & 1, (kt + 1) * BK);
    __syncthreads();
  };
  auto tail_step = [&](auto slot_c, int kt, bool store_next) {
    constexpr int slot = decltype(slot_c)::value;
    compute(slot & 1);
    if (store_next) sstore(IC<(slot + 1) % DEPTH>{}, (slot + 1) & 1, (kt + 1) * BK);
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
  if constexpr (sizeof(TO) == 2)
    epilogue_staged_f16<TE, MTM, MTN, WTM, WTN, SYM, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane, smem);
  else
    epilogue<MTM, MTN, WTM, WTN, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane);
}

template <typename TE, bool SYM, bool CHECKS>
hipError_t dispatch_f16(GemmArgs& a, dash_prec out_prec, bool y_sym, hipStream_t stream) {
  // 256-wide tiles: the kernel that reads an exactly symmetric right operand's columns as rows, or
  // the one that transposes a general right operand while staging it (no operand maps)
  const bool maps = a.p0.map_x || a.p0.map_y || (a.nprob > 1 && (a.p1.map_x || a.p1.map_y));
  const bool frz = a.p0.freeze || (a.nprob > 1 && a.p1.freeze);
  const int tile = (a.B % 256 == 0 && (y_sym || (!maps && !frz))) ? 256 : (a.B % 128 == 0 ? 128 : 64);
  a.tdim = a.B / tile;
  a.tiles = SYM ? a.tdim * (a.tdim + 1) / 2 : a.tdim * a.tdim;
  const bool half_out = out_prec != DASH_FP32;  // 2-byte output in the operand format
  // eight waves (two per SIMD: one wave's barrier and LDS latency are hidden behind the other's
  // MFMAs)
  // launches that carry stopped blocks of an adaptive solve (triangle-only products only)
  if constexpr (SYM) {
    if (frz) {
      if (tile == 256)  // frz launches take 256-wide tiles only with a symmetric right operand
        return half_out ? launch_interleaved(gemm_f16_ysym_kernel<TE, SYM, TE, CHECKS, 8, true>, a, stream, 512)
                        : launch_interleaved(gemm_f16_ysym_kernel<TE, SYM, float, CHECKS, 8, true>, a, stream, 512);
      if (tile == 128)
        return half_out ? launch_interleaved(gemm_f16_kernel<TE, 128, SYM, TE, CHECKS, true>, a, stream)
                        : launch_interleaved(gemm_f16_kernel<TE, 128, SYM, float, CHECKS, true>, a, stream);
      return half_out ? launch_interleaved(gemm_f16_kernel<TE, 64, SYM, TE, CHECKS, true>, a, stream)
                      : launch_interleaved(gemm_f16_kernel<TE, 64, SYM, float, CHECKS, true>, a, stream);
    }
  }
  if (tile == 256 && !y_sym)
    return half_out ? launch(gemm_f16_big_kernel<TE, SYM, TE, CHECKS>, a, stream)
                    : launch(gemm_f16_big_kernel<TE, SYM, float, CHECKS>, a, stream);
  if (tile == 256)
    return half_out ? launch(gemm_f16_ysym_kernel<TE, SYM, TE, CHECKS, 8>, a, stream, 512)
                    : launch(gemm_f16_ysym_kernel<TE, SYM, float, CHECKS, 8>, a, stream, 512);
  if (tile == 128)
    return half_out ? launch(gemm_f16_kernel<TE, 128, SYM, TE, CHECKS>, a, stream)
                    : launch(gemm_f16_kernel<TE, 128, SYM, float, CHECKS>, a, stream);
  return half_out ? launch(gemm_f16_kernel<TE, 64, SYM, TE, CHECKS>, a, stream)
                  : launch(gemm_f16_kernel<TE, 64, SYM, float, CHECKS>, a, stream);
}

}  // namespace

hipError_t launch_f16(GemmArgs& a, dash_prec in_prec, dash_prec out_prec, bool sym, bool y_sym, hipStream_t stream) {
  const bool checks = wants_checks(a.epi);
  if (in_prec == DASH_BF16) {
    if (checks)
      return sym ? dispatch_f16<__bf16, true, true>(a, out_prec, y_sym, stream)
                 : dispatch_f16<__bf16, false, true>(a, out_prec, y_sym, stream);
    return sym ? dispatch_f16<__bf16, true, false>(a, out_prec, y_sym, stream)
               : dispatch_f16<__bf16, false, false>(a, out_prec, y_sym, stream);
  }
  if (checks)
    return sym ? dispatch_f16<_Float16, true, true>(a, out_prec, y_sym, stream)
               : dispatch_f16<_Float16, false, true>(a, out_prec, y_sym, stream);
  return sym ? dispatch_f16<_Float16, true, false>(a, out_prec, y_sym, stream)
             : dispatch_f16<_Float16, false, false>(a, out_prec, y_sym, stream);
}

}  // namespace gemm
}  // namespace dash
