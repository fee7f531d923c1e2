// gemm_common.hpp -- pieces shared by the batched-product kernels (gemm_f32.hip, gemm_f16.hip):
// launch arguments, the XCD-aware workgroup -> (problem, block, tile) map and the fused epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include "dash_internal.hpp"

namespace dash {
namespace gemm {


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

// Shared epilogue for a wave holding MTM x MTN accumulators of 32 x 32 (layout of the 32x32 MFMA
// family: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32).
//
//   D  = alpha acc + beta C + delta E + gamma I,   D2 = alpha2 acc + gamma2 I   (per-block coefficients)
//
// SYM (triangle-only products): only tiles ti <= tj run, and within a diagonal tile only i <= j is
// kept.  Each kept element is stored at (i, j) directly and at (j, i) through LDS: the values are
// written transposed into `smem` and read back row by row, so the mirrored stores are as coalesced
// as the direct ones.  When the whole transposed tile fits in `smem` (ONE_PASS) it is filled while
// D is stored; otherwise the tile is mirrored in passes of R rows from D's values kept in acc, and
// a second output D2 is then re-derived from D, which requires alpha = 1, gamma = 0 and no C/E
// (enforced on the host).  The monitor counts off-diagonal kept elements twice under SYM.
template <int MTM, int MTN, int WTM, int WTN, bool SYM, typename TO, bool HAS_CE, int TILE, int SMEM_BYTES>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                         f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane, char* smem) {
  constexpr bool ONE_PASS = TILE * (TILE + 1) * (int)sizeof(TO) <= SMEM_BYTES;
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
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const bool diag_tile = SYM && tc.ti == tc.tj;
  TO* T = (TO*)smem;
  const int nthreads = blockDim.x;
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
        const int i = i0 + wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = j0 + wn * WTN + nt * 32 + li;
        const int64_t idx = (int64_t)i * B + j;
        cv[nt][r] = (HAS_CE && C) ? C[idx] : 0.f;
        ev[nt][r] = (HAS_CE && E) ? E[idx] : 0.f;
      }
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int jl = wn * WTN + nt * 32 + li;
        const int i = i0 + il, j = j0 + jl;
        const float x = acc[mt][nt][r];
        float v = al * x + be * cv[nt][r] + de * ev[nt][r];
        if (i == j) v += ga;
        if (SYM && ONE_PASS) T[jl * (TILE + 1) + il] = cvt_out<TO>(v);
        if (SYM && !ONE_PASS) acc[mt][nt][r] = v;
        if (diag_tile && i > j) continue;
        const int64_t idx = (int64_t)i * B + j;
        D[idx] = cvt_out<TO>(v);
        bad |= !isfinite(v);
        if (D2) {
          const float v2 = al2 * x + (i == j ? ga2 : 0.f);
          D2[idx] = cvt_out<TO>(v2);
          bad |= !isfinite(v2);
        }
        if (e.monitor) {
          const float dd = v - (i == j ? 1.f : 0.f);
          mon += (SYM && i != j) ? 2.f * dd * dd : dd * dd;
        }
      }
  }
  if (e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (e.status && bad) atomicOr(&e.status[b], 2);
  if (!SYM) return;

  if (ONE_PASS) {
    for (int out = 0; out < (D2 ? 2 : 1); ++out) {
      if (out) {  // refill the staging tile with D2's values (acc still holds the products)
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
          for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int il = wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              const int jl = wn * WTN + nt * 32 + li;
              const float v2 = al2 * acc[mt][nt][r] + (il + i0 == jl + j0 ? ga2 : 0.f);
              T[jl * (TILE + 1) + il] = cvt_out<TO>(v2);
            }
      }
      __syncthreads();
      TO* Dst = out ? D2 : D;
      for (int g = threadIdx.x; g < TILE * TILE; g += nthreads) {
        const int jl = g / TILE, il = g - jl * TILE;
        if (diag_tile && il >= jl) continue;  // only the strict lower part is a mirror
        Dst[(int64_t)(j0 + jl) * B + i0 + il] = T[jl * (TILE + 1) + il];
      }
    }
    return;
  }

  // multi-pass mirror: pass p covers tile rows [p R, p R + R), stored transposed T[jl][il - p R]
  constexpr int R0 = SMEM_BYTES / (int)sizeof(TO) / TILE - 1;  // largest R with TILE (R+1) fitting
  constexpr int R = R0 >= TILE / 2 ? TILE / 2 : (R0 >= TILE / 4 ? TILE / 4 : TILE / 8);
  static_assert(ONE_PASS || TILE * (R + 1) * (int)sizeof(TO) <= SMEM_BYTES, "mirror staging does not fit");
  constexpr int PASSES = TILE / R;
  for (int out = 0; out < (D2 ? 2 : 1); ++out) {
    TO* Dst = out ? D2 : D;
    for (int p = 0; p < PASSES; ++p) {
      __syncthreads();  // LDS is free: the main loop or the previous read-back is done
#pragma unroll
      for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
        for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const int jl = wn * WTN + nt * 32 + li;
            if (il / R != p) continue;
            const float v = acc[mt][nt][r];
            const float w = out ? al2 * v + (il + i0 == jl + j0 ? ga2 : 0.f) : v;
            T[jl * (R + 1) + (il - p * R)] = cvt_out<TO>(w);
          }
      __syncthreads();
      for (int g = threadIdx.x; g < TILE * R; g += nthreads) {
        const int jl = g / R, c = g - jl * R;
        const int il = p * R + c;
        if (diag_tile && il >= jl) continue;
        Dst[(int64_t)(j0 + jl) * B + i0 + il] = T[jl * (R + 1) + c];
      }
    }
  }
}

// Epilogue for binary16 outputs (no C/E operands, no second output): the tile is staged in LDS
// (row pitch TILE + 8 halves) and written back with 16-byte row stores instead of one 2-byte store
// per element.  SYM: a diagonal tile is made exactly symmetric inside LDS (each kept upper element
// is written at (i, j) and (j, i)) and stored in one pass; an off-diagonal tile is stored, then
// staged again transposed -- from the binary16 values packed in registers during the first pass,
// so the accumulators are read once -- and stored at (tj, ti).  Monitor and status as in `epilogue`.
// smem: TILE * (TILE + 8) halves.
template <int MTM, int MTN, int WTM, int WTN, bool SYM, int TILE>
__device__ __forceinline__ void epilogue_staged_f16(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                                    const f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane,
                                                    char* smem) {
  constexpr int PITCH = TILE + 8;
  const Epilogue& e = a.epi;
  const int B = a.B;
  const int64_t b = tc.b;
  const int64_t off = b * (int64_t)B * B;
  const float al = e.alpha * coef_of(e, e.ia, b);
  const float ga = e.gamma * coef_of(e, e.ig, b);
  const int li = lane & 31, h = lane >> 5;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const bool diag_tile = SYM && tc.ti == tc.tj;
  _Float16* S = (_Float16*)smem;
  _Float16* Dst = (_Float16*)P.D + off;
  const int nthreads = blockDim.x;
  float mon = 0.f;
  bool bad = false;
  uint32_t pk[MTM][MTN][8];  // the staged values, two halves per register (rows r and r + 1)

  auto store_tile = [&](int r0, int c0) {
    __syncthreads();
    for (int g = threadIdx.x; g < TILE * TILE / 8; g += nthreads) {
      const int row = g / (TILE / 8), c8 = g - row * (TILE / 8);
      *(f16x8*)(Dst + (int64_t)(r0 + row) * B + c0 + 8 * c8) = *(const f16x8*)&S[row * PITCH + 8 * c8];
    }
  };

  // pass 0: tile (ti, tj)
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int jl = wn * WTN + nt * 32 + li;
        const bool on_diag = (i0 + il == j0 + jl);
        const float v = al * acc[mt][nt][r] + (on_diag ? ga : 0.f);
        const _Float16 hv = (_Float16)v;
        const uint32_t bits = (uint32_t)__builtin_bit_cast(uint16_t, hv);
        if (r & 1)
          pk[mt][nt][r >> 1] |= bits << 16;
        else
          pk[mt][nt][r >> 1] = bits;
        if (diag_tile) {
          if (il > jl) continue;
          S[il * PITCH + jl] = hv;
          S[jl * PITCH + il] = hv;
        } else {
          S[il * PITCH + jl] = hv;
        }
        bad |= !isfinite(v);
        if (e.monitor) {
          const float dd = v - (on_diag ? 1.f : 0.f);
          mon += (SYM && !on_diag) ? 2.f * dd * dd : dd * dd;
        }
      }
  store_tile(i0, j0);
  if (SYM && !diag_tile) {  // pass 1: the mirror tile (tj, ti) from the packed values
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
      for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int jl = wn * WTN + nt * 32 + li;
          const uint16_t bits = (uint16_t)((r & 1) ? (pk[mt][nt][r >> 1] >> 16) : (pk[mt][nt][r >> 1] & 0xffffu));
          S[jl * PITCH + il] = __builtin_bit_cast(_Float16, bits);
        }
    store_tile(j0, i0);
  }
  if (e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (e.status && bad) atomicOr(&e.status[b], 2);
}

template <typename K>
hipError_t launch(K kernel, const GemmArgs& a, hipStream_t stream, int threads = 256) {
  const int64_t grid = (int64_t)a.nprob * a.N * a.tiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// kernel launchers of the two precisions
hipError_t launch_f32(GemmArgs& a, Trans trans, bool sym, hipStream_t stream);
hipError_t launch_f16(GemmArgs& a, dash_prec out_prec, bool sym, hipStream_t stream);

}  // namespace gemm
}  // namespace dash
