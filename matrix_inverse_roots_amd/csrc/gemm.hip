// gemm.hip -- batched B x B products on CDNA4 matrix cores (MFMA) with fused epilogues.
//
// Every solver step of the inverse-root iterations is a product of two B x B blocks, done for all
// N blocks of the stack at once ([PT] Metodologia, item 1: the whole stack goes through batched
// matrix products).  One launch covers one or two batched products (grid = problems x blocks x
// tiles) and fuses the affine combination the iteration needs, D = a*acc + b*C + d*E + g*I, with
// per-block coefficients read on the device.
//
// fp32 path: v_mfma_f32_32x32x2f32.  Workgroup = 4 waves (256 threads), macro tile TILE x TILE
// (128, or 64 when B is not a multiple of 128), wave tile (TILE/2)^2, k-step 32, LDS double buffer
// with register prefetch of the next k-slice.  Within one k-step, lane half h of an MFMA takes
// k = h*16 + s at step s, so each lane reads 16 consecutive k of its X row with 128-bit LDS loads;
// the Y operand is a single float per lane read straight from a row of the Y tile.
//
// fp16 path: v_mfma_f32_32x32x16_f16 (fp16 operands, fp32 accumulation), k-step 64; the Y tile is
// stored transposed in LDS so that both operands are read as 8 consecutive k per lane.
//
// Workgroup ids are remapped so that the tiles of one product run on one XCD (blocks are assigned
// round-robin to the 8 XCDs; consecutive logical ids then share that XCD's L2).
#include <hip/hip_runtime.h>

#include "dash_internal.hpp"

namespace dash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct GemmArgs {
  Product p0, p1;
  int nprob;
  int64_t N;
  int B;
  int tiles;  // tiles per product (all tiles, or the upper triangle when sym)
  int tdim;   // B / TILE
  Epilogue epi;
};

__device__ __forceinline__ float coef_of(const Epilogue& e, int idx, int64_t b) {
  return idx >= 0 ? e.coef[b * COEF_STRIDE + idx] : 1.f;
}

// Logical id for hardware workgroup w of G: workgroups are dealt to XCDs round-robin (w % 8), so
// give XCD x a contiguous range of logical ids.  A bijection on [0, G).
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t G) {
  const int64_t x = w & 7, slot = w >> 3;
  const int64_t q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + slot;
}

struct TileCoord {
  int prob;
  int64_t b;
  int ti, tj;
};

__device__ __forceinline__ TileCoord decode_tile(const GemmArgs& a, bool sym) {
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_prob = a.N * a.tiles;
  TileCoord c;
  c.prob = (int)(lid / per_prob);
  const int64_t rem = lid - (int64_t)c.prob * per_prob;
  c.b = rem / a.tiles;
  int t = (int)(rem - c.b * a.tiles);
  if (sym) {
    int ti = 0;
    while (t >= a.tdim - ti) {
      t -= a.tdim - ti;
      ++ti;
    }
    c.ti = ti;
    c.tj = ti + t;
  } else {
    c.ti = t / a.tdim;
    c.tj = t - c.ti * a.tdim;
  }
  return c;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename TO>
__device__ __forceinline__ TO cvt_out(float v) {
  return (TO)v;
}

// Shared epilogue for a wave holding MT x MT accumulators of 32 x 32 (layout of the 32x32 MFMA
// family: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32).
template <int MTM, int MTN, int WTM, int WTN, bool SYM, typename TO, bool HAS_CE = true>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                         const f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane, int TILE) {
  const Epilogue& e = a.epi;
  const int B = a.B;
  const int64_t b = tc.b;
  const int64_t off = b * (int64_t)B * B;
  const float al = e.alpha * coef_of(e, e.ia, b);
  const float be = e.beta * coef_of(e, e.ib, b);
  const float de = e.delta * coef_of(e, e.id, b);
  const float ga = e.gamma * coef_of(e, e.ig, b);
  const float al2 = e.alpha2 * coef_of(e, e.ia2, b);
  const float ga2 = e.gamma2 * coef_of(e, e.ig2, b);
  TO* D = (TO*)P.D + off;
  TO* D2 = P.D2 ? (TO*)P.D2 + off : nullptr;
  const float* C = P.C ? P.C + off : nullptr;
  const float* E = P.E ? P.E + off : nullptr;
  const int li = lane & 31, h = lane >> 5;
  float mon = 0.f;
  bool bad = false;
  // One row of MFMA tiles at a time: all C/E loads of the chunk are issued before any store, so
  // their latency is paid once per chunk (D may alias E: a lane reads and writes only its own
  // elements, so loading the chunk first is still exact).
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt) {
    float cv[MTN][16], ev[MTN][16];
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = tc.ti * TILE + wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = tc.tj * TILE + wn * WTN + nt * 32 + li;
        const int64_t idx = (int64_t)i * B + j;
        cv[nt][r] = (HAS_CE && C) ? C[idx] : 0.f;
        ev[nt][r] = (HAS_CE && E) ? E[idx] : 0.f;
      }
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = tc.ti * TILE + wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = tc.tj * TILE + wn * WTN + nt * 32 + li;
        if (SYM && tc.ti == tc.tj && i > j) continue;
        const int64_t idx = (int64_t)i * B + j;
        const float x = acc[mt][nt][r];
        float v = al * x + be * cv[nt][r] + de * ev[nt][r];
        if (i == j) v += ga;
        D[idx] = cvt_out<TO>(v);
        if (SYM && i != j) D[(int64_t)j * B + i] = cvt_out<TO>(v);
        bad |= !isfinite(v);
        if (D2) {
          const float v2 = al2 * x + (i == j ? ga2 : 0.f);
          D2[idx] = cvt_out<TO>(v2);
          bad |= !isfinite(v2);
        }
        if (e.monitor) {
          const float dd = v - (i == j ? 1.f : 0.f);
          mon += dd * dd;
        }
      }
  }
  if (e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (e.status && bad) atomicOr(&e.status[b], 2);
}

// ------------------------------------------------------------------------------------------------
// fp32 operands
// ------------------------------------------------------------------------------------------------
template <int TILE, int TX, int TY, bool SYM, typename TO>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BK = 32;
  constexpr int WT = TILE / 2;
  constexpr int MT = WT / 32;
  constexpr int LDA = BK + 4;    // As[m][k]
  constexpr int LDB = TILE + 4;  // Bs[k][n]
  constexpr int NL = TILE * BK / 4 / 256;
  __shared__ __attribute__((aligned(16))) float As[2][TILE * LDA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

  const TileCoord tc = decode_tile(a, SYM);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const float* X = (const float*)P.X + off;
  const float* Y = (const float*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  f32x4 ra[NL], rb[NL];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      if (!TX) {
        const int row = f / (BK / 4), c4 = f % (BK / 4);
        ra[r] = *(const f32x4*)(X + (int64_t)(i0 + row) * B + k0 + 4 * c4);
      } else {  // X[i][k] = G[k][i]
        const int krow = f / (TILE / 4), c4 = f % (TILE / 4);
        ra[r] = *(const f32x4*)(X + (int64_t)(k0 + krow) * B + i0 + 4 * c4);
      }
      if (!TY) {
        const int krow = f / (TILE / 4), c4 = f % (TILE / 4);
        rb[r] = *(const f32x4*)(Y + (int64_t)(k0 + krow) * B + j0 + 4 * c4);
      } else {  // Y[k][j] = G[j][k]
        const int row = f / (BK / 4), c4 = f % (BK / 4);
        rb[r] = *(const f32x4*)(Y + (int64_t)(j0 + row) * B + k0 + 4 * c4);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      if (!TX) {
        const int row = f / (BK / 4), c4 = f % (BK / 4);
        *(f32x4*)&As[buf][row * LDA + 4 * c4] = ra[r];
      } else {
        const int krow = f / (TILE / 4), c4 = f % (TILE / 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) As[buf][(4 * c4 + q) * LDA + krow] = ra[r][q];
      }
      if (!TY) {
        const int krow = f / (TILE / 4), c4 = f % (TILE / 4);
        *(f32x4*)&Bs[buf][krow * LDB + 4 * c4] = rb[r];
      } else {
        const int row = f / (BK / 4), c4 = f % (BK / 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[buf][(4 * c4 + q) * LDB + row] = rb[r][q];
      }
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
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      f32x4 av[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = *(const f32x4*)&as[(wm * WT + mt * 32 + li) * LDA + h * 16 + 4 * s4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = h * 16 + 4 * s4 + q;
        float bv[MT];
#pragma unroll
        for (int nt = 0; nt < MT; ++nt) bv[nt] = bs[kk * LDB + wn * WT + nt * 32 + li];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < MT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt][q], bv[nt], acc[mt][nt], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<MT, MT, WT, WT, SYM, TO>(a, tc, P, acc, wm, wn, lane, TILE);
}

// ------------------------------------------------------------------------------------------------
// fp16 operands, fp32 accumulation
// ------------------------------------------------------------------------------------------------
template <int TILE, typename TO>
__global__ __launch_bounds__(256) void gemm_f16_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int WT = TILE / 2;
  constexpr int MT = WT / 32;
  constexpr int LD = BK + 8;  // As[m][k], Bs[n][k] (Y tile transposed)
  constexpr int NL = TILE * BK / 8 / 256;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][TILE * LD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][TILE * LD];

  const TileCoord tc = decode_tile(a, false);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const _Float16* X = (const _Float16*)P.X + off;
  const _Float16* Y = (const _Float16*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  f16x8 ra[NL], rb[NL];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      ra[r] = *(const f16x8*)(X + (int64_t)(i0 + row) * B + k0 + 8 * c8);
      const int krow = f / (TILE / 8), n8 = f % (TILE / 8);
      rb[r] = *(const f16x8*)(Y + (int64_t)(k0 + krow) * B + j0 + 8 * n8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int f = tid + 256 * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      *(f16x8*)&As[buf][row * LD + 8 * c8] = ra[r];
      const int krow = f / (TILE / 8), n8 = f % (TILE / 8);
#pragma unroll
      for (int q = 0; q < 8; ++q) Bs[buf][(8 * n8 + q) * LD + krow] = rb[r][q];
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
    const _Float16* as = As[buf];
    const _Float16* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 av[MT], bv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = *(const f16x8*)&as[(wm * WT + mt * 32 + li) * LD + h * 32 + 8 * s];
#pragma unroll
      for (int nt = 0; nt < MT; ++nt) bv[nt] = *(const f16x8*)&bs[(wn * WT + nt * 32 + li) * LD + h * 32 + 8 * s];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < MT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<MT, MT, WT, WT, false, TO>(a, tc, P, acc, wm, wn, lane, TILE);
}


// ------------------------------------------------------------------------------------------------
// fp16 operands, 256 x 256 macro tile (B % 256 == 0).  Four waves as 2 x 2, wave tile 128 x 128
// (4 x 4 accumulators of 32 x 32, held in the accumulation registers at one wave per SIMD).  Every
// thread stages 8 pieces of the X slice (256 rows x 64 k, 16-byte loads) and one 8 (k) x 8 (n)
// sub-block of the Y slice, loaded as eight 16-byte row pieces and transposed in registers, so both
// LDS tiles hold rows of 64 consecutive k.  LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
// (row ^ row/8) & 7, which keeps both the MFMA reads (8 consecutive rows, one chunk) and the
// transposed writes (rows 8 apart, one chunk) free of bank conflicts.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ (row ^ (row >> 3))) & 7; }

template <typename TO>
__global__ __launch_bounds__(256) void gemm_f16_big_kernel(GemmArgs a) {
  constexpr int TILE = 256, BK = 64, MT = 4, WT = 128;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][TILE * BK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][TILE * BK];

  const TileCoord tc = decode_tile(a, false);
  const Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const _Float16* X = (const _Float16*)P.X + off;
  const _Float16* Y = (const _Float16*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;
  const int kb = tid >> 5, nb = tid & 31;  // this thread's 8 x 8 sub-block of the Y slice

  // X slice: 8 pieces of 16 bytes, piece c = tid + 256 r -> row c / 8, chunk c % 8.
  // Y slice: k rows 8 kb .. 8 kb + 7, n columns 8 nb .. 8 nb + 7, transposed in registers.
  f16x8 lx[8], ly[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = tid + 256 * r;
      lx[r] = *(const f16x8*)(X + (int64_t)(i0 + (c >> 3)) * B + k0 + 8 * (c & 7));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ly[q] = *(const f16x8*)(Y + (int64_t)(k0 + 8 * kb + q) * B + j0 + 8 * nb);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = tid + 256 * r;
      const int row = c >> 3;
      *(f16x8*)&As[buf][row * BK + 8 * swz(row, c & 7)] = lx[r];
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      f16x8 col;
#pragma unroll
      for (int q = 0; q < 8; ++q) col[q] = ly[q][n];
      const int row = 8 * nb + n;
      *(f16x8*)&Bs[buf][row * BK + 8 * swz(row, kb)] = col;
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
    const _Float16* as = As[buf];
    const _Float16* bs = Bs[buf];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 4 * h + s;
      f16x8 av[MT], bv[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = wm * WT + mt * 32 + li;
        av[mt] = *(const f16x8*)&as[row * BK + 8 * swz(row, chunk)];
      }
#pragma unroll
      for (int nt = 0; nt < MT; ++nt) {
        const int row = wn * WT + nt * 32 + li;
        bv[nt] = *(const f16x8*)&bs[row * BK + 8 * swz(row, chunk)];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < MT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  epilogue<MT, MT, WT, WT, false, TO, false>(a, tc, P, acc, wm, wn, lane, TILE);
}

template <typename K>
hipError_t launch(K kernel, const GemmArgs& a, hipStream_t stream, int threads = 256) {
  const int64_t grid = (int64_t)a.nprob * a.N * a.tiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <int TILE>
hipError_t dispatch(GemmArgs& a, dash_prec in_prec, dash_prec out_prec, Trans trans, bool sym,
                    hipStream_t stream) {
  a.tdim = a.B / TILE;
  a.tiles = sym ? a.tdim * (a.tdim + 1) / 2 : a.tdim * a.tdim;
  if (in_prec == DASH_FP32) {
    if (out_prec != DASH_FP32) return hipErrorInvalidValue;
    if (trans == Trans::NN) {
      if (sym) return launch(gemm_f32_kernel<TILE, 0, 0, true, float>, a, stream);
      return launch(gemm_f32_kernel<TILE, 0, 0, false, float>, a, stream);
    }
    if (!sym) return hipErrorInvalidValue;
    if (trans == Trans::NT) return launch(gemm_f32_kernel<TILE, 0, 1, true, float>, a, stream);
    return launch(gemm_f32_kernel<TILE, 1, 0, true, float>, a, stream);
  }
  if (trans != Trans::NN || sym) return hipErrorInvalidValue;
  if (out_prec == DASH_FP16) return launch(gemm_f16_kernel<TILE, _Float16>, a, stream);
  return launch(gemm_f16_kernel<TILE, float>, a, stream);
}

}  // namespace

hipError_t launch_gemm(const Product* probs, int nprob, int64_t N, int B, dash_prec in_prec, dash_prec out_prec,
                       Trans trans, bool sym, const Epilogue& epi, hipStream_t stream) {
  if (nprob < 1 || nprob > 2 || N < 1 || B % 64 != 0) return hipErrorInvalidValue;
  GemmArgs a;
  a.p0 = probs[0];
  a.p1 = nprob > 1 ? probs[1] : probs[0];
  a.nprob = nprob;
  a.N = N;
  a.B = B;
  a.epi = epi;
  if (in_prec == DASH_FP16 && B % 256 == 0 && trans == Trans::NN && !sym) {
    a.tdim = B / 256;
    a.tiles = a.tdim * a.tdim;
    if (out_prec == DASH_FP16) return launch(gemm_f16_big_kernel<_Float16>, a, stream);
    return launch(gemm_f16_big_kernel<float>, a, stream);
  }
  if (B % 128 == 0) return dispatch<128>(a, in_prec, out_prec, trans, sym, stream);
  return dispatch<64>(a, in_prec, out_prec, trans, sym, stream);
}

}  // namespace dash
