// vec.hip -- 1-D parameters: a vector gradient is cut into pieces of B, each piece keeps the B x B
// statistic L <- beta L + (1 - beta) g g^T, and its update is L^{-1/2} g (the exponent -1/(2k) of a
// Shampoo preconditioner for an order-k tensor, k = 1).  These kernels move HBM only: the pieces'
// copies, the rank-one statistic update and the block-times-vector apply.
#include <hip/hip_runtime.h>

#include "dash_internal.hpp"

namespace dash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// pieces[e] = v[e] for e < len, 0 up to the end of the last piece (to_pieces); or v[e] = pieces[e]
// for e < len (back).
template <bool TO_PIECES>
__global__ __launch_bounds__(256) void vec_copy_kernel(float* v, int64_t len, float* pieces, int64_t total) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (TO_PIECES) {
    if (e < total) pieces[e] = e < len ? v[e] : 0.f;
  } else {
    if (e < len) v[e] = pieces[e];
  }
}

// L_p <- beta L_p + (1 - beta) g_p g_p^T.  Workgroup: 16 rows of one piece, 256 threads; each thread
// streams float4 columns of its rows.  (1 - beta) (g_i g_j) is the same fp32 value at (i, j) and
// (j, i), so a symmetric L stays exactly symmetric.
constexpr int VROWS = 16;
__global__ __launch_bounds__(256) void vec_stats_kernel(const float* g, int B, float beta, float* L) {
  const int chunks = B / VROWS;
  const int64_t p = blockIdx.x / chunks;
  const int r0 = (int)(blockIdx.x - p * chunks) * VROWS;
  const float* gp = g + p * (int64_t)B;
  float* Lp = L + p * (int64_t)B * B;
  const float c = 1.f - beta;
  const int c4n = B / 4;  // float4 per row
  for (int f = threadIdx.x; f < VROWS * c4n; f += 256) {
    const int row = r0 + f / c4n, c4 = f % c4n;
    const float gi = gp[row];
    const f32x4 gj = *(const f32x4*)(gp + 4 * c4);
    f32x4* lp = (f32x4*)(Lp + (int64_t)row * B + 4 * c4);
    f32x4 l = *lp;
#pragma unroll
    for (int q = 0; q < 4; ++q) l[q] = fmaf(beta, l[q], c * (gi * gj[q]));
    *lp = l;
  }
}

// u_p = X_p g_p.  Workgroup: 64 rows of one piece, 4 waves of 16 rows; g_p staged in LDS; each wave
// reads a row 1 KiB at a time and reduces its dot product across the wave.
__global__ __launch_bounds__(256) void vec_apply_kernel(const float* X, const float* g, int B, float* u) {
  extern __shared__ __attribute__((aligned(16))) float gs[];
  const int chunks = B / 64;
  const int64_t p = blockIdx.x / chunks;
  const int r0 = (int)(blockIdx.x - p * chunks) * 64;
  const float* gp = g + p * (int64_t)B;
  for (int e = threadIdx.x; e < B; e += 256) gs[e] = gp[e];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* Xp = X + p * (int64_t)B * B;
  for (int rr = 0; rr < 16; ++rr) {
    const int row = r0 + wave * 16 + rr;
    const float* xr = Xp + (int64_t)row * B;
    float acc = 0.f;
    for (int c = 4 * lane; c < B; c += 256) {
      const f32x4 x = *(const f32x4*)(xr + c);
      const f32x4 gv = *(const f32x4*)(gs + c);
      acc += x[0] * gv[0] + x[1] * gv[1] + x[2] * gv[2] + x[3] * gv[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) u[p * (int64_t)B + row] = acc;
  }
}

}  // namespace

hipError_t launch_vec_copy(float* v, int64_t len, float* pieces, int B, bool to_pieces, hipStream_t stream) {
  const int64_t total = (len + B - 1) / B * B;
  const int64_t n = to_pieces ? total : len;
  const int64_t grid = (n + 255) / 256;
  if (grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (to_pieces)
    hipLaunchKernelGGL(vec_copy_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, v, len, pieces, total);
  else
    hipLaunchKernelGGL(vec_copy_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, v, len, pieces, total);
  return hipGetLastError();
}

hipError_t launch_vec_stats(const float* g, int64_t P, int B, float beta, float* L, hipStream_t stream) {
  const int64_t grid = P * (B / VROWS);
  if (B % 64 != 0 || grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vec_stats_kernel, dim3((unsigned)grid), dim3(256), 0, stream, g, B, beta, L);
  return hipGetLastError();
}

hipError_t launch_vec_apply(const float* X, const float* g, int64_t P, int B, float* u, hipStream_t stream) {
  const int64_t grid = P * (B / 64);
  if (B % 64 != 0 || grid < 1 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vec_apply_kernel, dim3((unsigned)grid), dim3(256), (size_t)B * sizeof(float), stream, X, g, B,
                     u);
  return hipGetLastError();
}

}  // namespace dash
