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

template <typename K>
hipError_t launch(K kernel, const GemmArgs& a, hipStream_t stream, int threads = 256) {
  const int64_t grid = (int64_t)a.nprob * a.N * a.tiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// kernel launchers of the two precisions
hipError_t launch_f32(GemmArgs& a, Trans trans, bool sym, hipStream_t stream);
hipError_t launch_f16(GemmArgs& a, dash_prec out_prec, hipStream_t stream);

}  // namespace gemm
}  // namespace dash
