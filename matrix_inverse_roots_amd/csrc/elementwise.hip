// elementwise.hip -- HBM-bound kernels around the products: per-block coefficients, affine
// identity combinations (solver start terms, casts, unscaling), fills, per-block magnitude bounds,
// and stack/unstack copies.
//
// All of them stream 16-byte vectors with consecutive lanes on consecutive addresses.
#include <hip/hip_runtime.h>

#include "dash_internal.hpp"

namespace dash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// coef row of block b from s_b.  The roots are taken in double so that a power-of-two change of
// s changes every coefficient by the exact power of two (scale equivariance of the solvers).
__global__ void coef_kernel(const float* s, int64_t N, float* coef, int32_t* status) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= N) return;
  const float sv = s[b];
  float* c = coef + b * COEF_STRIDE;
  if (!(isfinite(sv) && sv > 0.f)) {
    const float nan = __builtin_nanf("");
    for (int q = 0; q < COEF_STRIDE; ++q) c[q] = nan;
    if (status) atomicOr(&status[b], 1);
    return;
  }
  const double sd = (double)sv;
  const double r1 = 1.0 / sd;
  const double u = 1.0 / sqrt(sqrt(sd));
  c[CO_R1] = (float)r1;
  c[CO_R2] = (float)(r1 * r1);
  c[CO_U] = (float)u;
  c[CO_SQ] = (float)sqrt(sd);
  c[CO_R1U] = (float)(r1 * u);
  c[CO_P2] = 1.f;
  c[CO_P2INV] = 1.f;
  c[CO_S] = sv;
  c[CO_RSQ] = (float)(1.0 / sqrt(sd));
  c[9] = 0.f;
}

__device__ __forceinline__ float co(const float* coef, int idx, int64_t b) {
  return idx >= 0 ? coef[b * COEF_STRIDE + idx] : 1.f;
}

__device__ __forceinline__ void store4(void* D, dash_prec p, int64_t e, f32x4 v) {
  if (p == DASH_FP32) {
    *(f32x4*)((float*)D + e) = v;
  } else if (p == DASH_BF16) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 bv;
    bv[0] = (__bf16)v[0];
    bv[1] = (__bf16)v[1];
    bv[2] = (__bf16)v[2];
    bv[3] = (__bf16)v[3];
    *(b4*)((__bf16*)D + e) = bv;
  } else {
    f16x4 hv;
    hv[0] = (_Float16)v[0];
    hv[1] = (_Float16)v[1];
    hv[2] = (_Float16)v[2];
    hv[3] = (_Float16)v[3];
    *(f16x4*)((_Float16*)D + e) = hv;
  }
}

// One workgroup = 256 threads x 4 vectors of 4 = 4096 consecutive elements of one block.
constexpr int AFF_CHUNK = 4096;

__global__ __launch_bounds__(256) void affine_kernel(Affine op, int64_t N, int B) {
  const int64_t chunks = (int64_t)B * B / AFF_CHUNK;
  const int64_t b = blockIdx.x / chunks;
  const int64_t c = blockIdx.x - b * chunks;
  const int64_t base = b * (int64_t)B * B + c * AFF_CHUNK;
  const float a = op.a * co(op.coef, op.ia, b), g = op.g * co(op.coef, op.ig, b);
  const float a2 = op.a2 * co(op.coef, op.ia2, b), g2 = op.g2 * co(op.coef, op.ig2, b);
  float mon = 0.f;
  bool bad = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t e = base + 4 * (threadIdx.x + 256 * r);   // element index within the stack
    const int64_t in_blk = e - b * (int64_t)B * B;
    const int row = (int)(in_blk / B), col = (int)(in_blk % B);
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (op.X) {
      if (op.x_prec == DASH_FP32) {
        x = *(const f32x4*)((const float*)op.X + e);
      } else if (op.x_prec == DASH_BF16) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        const b4 bx = *(const b4*)((const __bf16*)op.X + e);
        x = f32x4{(float)bx[0], (float)bx[1], (float)bx[2], (float)bx[3]};
      } else {
        const f16x4 hx = *(const f16x4*)((const _Float16*)op.X + e);
        x = f32x4{(float)hx[0], (float)hx[1], (float)hx[2], (float)hx[3]};
      }
    }
    f32x4 v, v2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool diag = (row == col + q);
      v[q] = (op.X ? a * x[q] : 0.f) + (diag ? g : 0.f);
      v2[q] = (op.X ? a2 * x[q] : 0.f) + (diag ? g2 : 0.f);
      bad |= !isfinite(v[q]);
      if (op.monitor) {
        const float d = v[q] - (diag ? 1.f : 0.f);
        mon += d * d;
      }
    }
    store4(op.D, op.d_prec, e, v);
    if (op.D2) {
      store4(op.D2, op.d2_prec, e, v2);
#pragma unroll
      for (int q = 0; q < 4; ++q) bad |= !isfinite(v2[q]);
    }
  }
  if (op.monitor) {
    mon = wave_sum(mon);
    if ((threadIdx.x & 63) == 0) atomicAdd(&op.monitor[b * op.mon_stride], op.mon_mul * mon);
  }
  if (op.status && bad) atomicOr(&op.status[b], 2);
}

// Affine map of the symmetric matrix built from the upper triangle of X (fp32):
// Xu[i][j] = X[min(i,j)][max(i,j)].  One workgroup per pair of 64 x 64 tiles (ti <= tj): the upper
// tile is staged in LDS and both it and its mirror are written, so D (and D2) come out exactly
// symmetric whatever the lower triangle of X holds.
__global__ __launch_bounds__(256) void sym_affine_kernel(Affine op, int64_t N, int B) {
  constexpr int T = 64;
  __shared__ float U[T][T + 1];
  const int nt = B / T;
  const int64_t pairs = (int64_t)nt * (nt + 1) / 2;
  const int64_t b = blockIdx.x / pairs;
  int t = (int)(blockIdx.x - b * pairs);
  int ti = 0;
  while (t >= nt - ti) {
    t -= nt - ti;
    ++ti;
  }
  const int tj = ti + t;
  const float* X = (const float*)op.X + b * (int64_t)B * B;
  const float a = op.a * co(op.coef, op.ia, b), g = op.g * co(op.coef, op.ig, b);
  const float a2 = op.a2 * co(op.coef, op.ia2, b), g2 = op.g2 * co(op.coef, op.ig2, b);
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // 64 x 64 floats = 1024 float4, 4 per thread
    const int f = threadIdx.x + 256 * q;
    const int r = f >> 4, c4 = f & 15;
    const f32x4 v = *(const f32x4*)(X + (int64_t)(ti * T + r) * B + tj * T + 4 * c4);
    U[r][4 * c4 + 0] = v[0];
    U[r][4 * c4 + 1] = v[1];
    U[r][4 * c4 + 2] = v[2];
    U[r][4 * c4 + 3] = v[3];
  }
  __syncthreads();
  float mon = 0.f;
  for (int m = 0; m < (ti == tj ? 1 : 2); ++m) {  // m = 0: tile (ti, tj); m = 1: its mirror (tj, ti)
    const int R0 = (m ? tj : ti) * T, C0 = (m ? ti : tj) * T;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = threadIdx.x + 256 * q;
      const int r = f >> 4, c4 = f & 15;
      f32x4 v, v2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 4 * c4 + e;
        // value at (R0 + r, C0 + c) from the upper triangle
        const float x = (m == 0 && (ti < tj || r <= c)) ? U[r][c] : U[c][r];
        const bool diag = (R0 + r == C0 + c);
        v[e] = a * x + (diag ? g : 0.f);
        v2[e] = a2 * x + (diag ? g2 : 0.f);
        if (op.monitor) {
          const float d = v[e] - (diag ? 1.f : 0.f);
          mon += d * d;
        }
      }
      const int64_t idx = b * (int64_t)B * B + (int64_t)(R0 + r) * B + C0 + 4 * c4;
      store4(op.D, op.d_prec, idx, v);
      if (op.D2) store4(op.D2, op.d2_prec, idx, v2);
    }
  }
  if (op.monitor) {
    mon = wave_sum(mon);
    if ((threadIdx.x & 63) == 0) atomicAdd(&op.monitor[b * op.mon_stride], op.mon_mul * mon);
  }
}

// out[b] = max |A_b| over the block's B^2 elements (NaN elements are passed over), one workgroup
// per block streaming 16-byte vectors
__global__ __launch_bounds__(512) void block_amax_kernel(const float* A, int B, float* out) {
  const int64_t b = blockIdx.x;
  const f32x4* a = (const f32x4*)(A + b * (int64_t)B * B);
  const int n4 = B * B / 4;
  float m = 0.f;
#pragma unroll 4
  for (int i = threadIdx.x; i < n4; i += 512) {
    const f32x4 v = a[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[8];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 8; ++w) m = fmaxf(m, red[w]);
    out[b] = m;
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void monitor_finish_kernel(float* m, int64_t n, float inv_sqrt_b) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) m[i] = sqrtf(m[i]) * inv_sqrt_b;
}

// stopping rule of the adaptive solvers (see launch_freeze_update)
__global__ void freeze_reset_kernel(int32_t* freeze, int32_t* steps, int steps_stride, int T, int64_t N) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= N) return;
  freeze[b] = 0;
  if (steps) steps[b * steps_stride] = T;
}

__global__ void freeze_update_kernel(const float* monitor, int mon_stride, int col, float inv_sqrt_b, float tol,
                                     int32_t* freeze, int32_t* steps, int steps_stride, int step, int64_t N) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= N || freeze[b]) return;
  const float m = sqrtf(monitor[b * mon_stride + col]) * inv_sqrt_b;
  if (m <= tol) {  // a NaN monitor never freezes: the block runs on and is flagged at the end
    freeze[b] = 1;
    if (steps) steps[b * steps_stride] = step;
  }
}

// Copy one weight's tiles to (to_stack) or from the stack.  Workgroup = 8 rows of one tile.
// Stack / unstack.  The stack side of a copy is one linear stream, so each workgroup moves
// COPY_VEC * 256 consecutive float4 of it and gathers them from (or scatters them to) the rows of
// the weight they belong to.  All loads of a thread are issued before its stores, and both are
// non-temporal: the data is streamed once and is far larger than the caches.  A launch covers up
// to COPY_GROUP weights; the weight of a workgroup comes from the prefix table in the arguments.
// Edge tiles of a weight whose sides are not multiples of B: the part outside the weight is zero
// in the stack and is not written back (a float4 that straddles the last column goes element by
// element).
constexpr int COPY_VEC = 4;

template <bool TO_STACK>
__global__ __launch_bounds__(256) void tile_copy_kernel(CopyGroup g, int B, float* stack) {
  const int wg = blockIdx.x;
  int wi = 0;
  while (wi + 1 < g.n && wg >= g.wg_base[wi + 1]) ++wi;
  const unsigned vpr = (unsigned)B / 4;  // float4 per tile row
  const int64_t total = (g.row_base[wi + 1] - g.row_base[wi]) * vpr;
  const int64_t q0 = (int64_t)(wg - g.wg_base[wi]) * (256 * COPY_VEC);
  const int64_t row0 = q0 / vpr;
  const unsigned c0 = (unsigned)(q0 - row0 * vpr);
  const int64_t t0 = row0 / B;
  const unsigned r0 = (unsigned)(row0 - t0 * B);
  const unsigned tiles_c = (unsigned)g.tiles_c[wi];
  const int64_t ld = g.ld[wi], rows = g.rows[wi], cols = g.cols[wi];
  f32x4* lin = (f32x4*)(stack + g.row_base[wi] * B) + q0;
  float* wp[COPY_VEC];
  int64_t col[COPY_VEC];
  bool in_rows[COPY_VEC];
  f32x4 v[COPY_VEC];
#pragma unroll
  for (int i = 0; i < COPY_VEC; ++i) {
    const unsigned d = i * 256 + threadIdx.x;
    const unsigned dr = (c0 + d) / vpr, c4 = c0 + d - dr * vpr;
    const unsigned rr = r0 + dr, tt = rr / (unsigned)B, r = rr - tt * (unsigned)B;
    const unsigned t = (unsigned)t0 + tt;  // tiles per weight < 2^31 (checked on the host)
    const unsigned tr = t / tiles_c, tc = t - tr * tiles_c;
    const int64_t grow = (int64_t)tr * B + r;
    col[i] = (int64_t)tc * B + 4 * c4;
    in_rows[i] = grow < rows;
    wp[i] = g.ptr[wi] + grow * ld + col[i];
  }
  if (rows % B == 0 && cols % B == 0) {  // no edge tiles in this weight
#pragma unroll
    for (int i = 0; i < COPY_VEC; ++i) {
      const unsigned d = i * 256 + threadIdx.x;
      if (q0 + d < total) v[i] = __builtin_nontemporal_load(TO_STACK ? (const f32x4*)wp[i] : lin + d);
    }
#pragma unroll
    for (int i = 0; i < COPY_VEC; ++i) {
      const unsigned d = i * 256 + threadIdx.x;
      if (q0 + d < total) __builtin_nontemporal_store(v[i], TO_STACK ? lin + d : (f32x4*)wp[i]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < COPY_VEC; ++i) {
    const unsigned d = i * 256 + threadIdx.x;
    if (q0 + d < total) {
      if (!TO_STACK) {
        v[i] = __builtin_nontemporal_load(lin + d);
      } else if (in_rows[i] && col[i] + 3 < cols) {
        v[i] = __builtin_nontemporal_load((const f32x4*)wp[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[i][e] = (in_rows[i] && col[i] + e < cols) ? wp[i][e] : 0.f;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < COPY_VEC; ++i) {
    const unsigned d = i * 256 + threadIdx.x;
    if (q0 + d >= total) continue;
    if (TO_STACK) {
      __builtin_nontemporal_store(v[i], lin + d);
    } else if (in_rows[i] && col[i] + 3 < cols) {
      __builtin_nontemporal_store(v[i], (f32x4*)wp[i]);
    } else if (in_rows[i]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col[i] + e < cols) wp[i][e] = v[i][e];
    }
  }
}

}  // namespace

hipError_t launch_coef(const float* s, int64_t N, float* coef, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(coef_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, s, N, coef, status);
  return hipGetLastError();
}

hipError_t launch_affine(const Affine& op, int64_t N, int B, hipStream_t stream) {
  const int64_t grid = N * ((int64_t)B * B / AFF_CHUNK);
  if ((int64_t)B * B % AFF_CHUNK != 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(affine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, op, N, B);
  return hipGetLastError();
}

hipError_t launch_sym_affine(const Affine& op, int64_t N, int B, hipStream_t stream) {
  const int nt = B / 64;
  const int64_t grid = N * (int64_t)nt * (nt + 1) / 2;
  if (B % 64 != 0 || op.x_prec != DASH_FP32 || !op.X || op.status || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sym_affine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, op, N, B);
  return hipGetLastError();
}

hipError_t launch_block_amax(const float* A, int64_t N, int B, float* out, hipStream_t stream) {
  if (N < 1 || N > 0x7fffffffLL || B % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_amax_kernel, dim3((unsigned)N), dim3(512), 0, stream, A, B, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

hipError_t launch_monitor_finish(float* monitor, int64_t n, int B, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(monitor_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, monitor, n,
                     (float)(1.0 / sqrt((double)B)));
  return hipGetLastError();
}

// Guarded correction: block b takes its candidate (accept[b] = 1) when the candidate's residual
// (monitor column q + 1, a sum of squares) is below the current one (column q); otherwise it stops
// correcting (freeze[b] = 1).  Stopped blocks are left alone.
__global__ void accept_kernel(const float* mon, int mon_stride, int q, int32_t* freeze, int32_t* accept, int64_t N) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= N) return;
  int32_t ok = 0;
  if (!freeze[b]) {
    ok = mon[b * mon_stride + q + 1] < mon[b * mon_stride + q];  // NaN compares false: stop
    if (!ok) freeze[b] = 1;
  }
  accept[b] = ok;
}

// dst[b] = src[b] for the blocks with accept[b] != 0
__global__ __launch_bounds__(256) void masked_copy_kernel(const float* src, float* dst, const int32_t* accept, int B) {
  const int64_t chunks = (int64_t)B * B / AFF_CHUNK;
  const int64_t b = blockIdx.x / chunks;
  if (!accept[b]) return;
  const int64_t base = b * (int64_t)B * B + (blockIdx.x - b * chunks) * AFF_CHUNK;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t e = base + 4 * (threadIdx.x + 256 * r);
    *(f32x4*)(dst + e) = *(const f32x4*)(src + e);
  }
}

hipError_t launch_accept(const float* mon, int mon_stride, int q, int32_t* freeze, int32_t* accept, const float* src,
                         float* dst, int64_t N, int B, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, mon, mon_stride, q,
                     freeze, accept, N);
  const int64_t grid = N * ((int64_t)B * B / AFF_CHUNK);
  if ((int64_t)B * B % AFF_CHUNK != 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(masked_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, accept, B);
  return hipGetLastError();
}

hipError_t launch_freeze_reset(int32_t* freeze, int32_t* steps, int steps_stride, int T, int64_t N,
                               hipStream_t stream) {
  hipLaunchKernelGGL(freeze_reset_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, freeze, steps,
                     steps_stride, T, N);
  return hipGetLastError();
}

hipError_t launch_freeze_update(const float* monitor, int mon_stride, int col, int B, float tol, int32_t* freeze,
                                int32_t* steps, int steps_stride, int step, int64_t N, hipStream_t stream) {
  hipLaunchKernelGGL(freeze_update_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, monitor,
                     mon_stride, col, (float)(1.0 / sqrt((double)B)), tol, freeze, steps, steps_stride, step, N);
  return hipGetLastError();
}

hipError_t launch_tile_copy(const dash_mat* w, int n, int B, float* stack, bool to_stack, hipStream_t stream) {
  const int64_t f4_per_wg = 256 * COPY_VEC;
  for (int i0 = 0; i0 < n; i0 += COPY_GROUP) {
    CopyGroup g{};
    g.n = n - i0 < COPY_GROUP ? n - i0 : COPY_GROUP;
    int64_t wgs = 0;
    g.row_base[0] = 0;
    g.wg_base[0] = 0;
    for (int j = 0; j < g.n; ++j) {
      const dash_mat& m = w[i0 + j];
      const int64_t tiles_r = (m.rows + B - 1) / B, tiles_c = (m.cols + B - 1) / B;
      const int64_t tiles = tiles_r * tiles_c;
      if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
      g.ptr[j] = m.ptr;
      g.ld[j] = m.ld;
      g.rows[j] = m.rows;
      g.cols[j] = m.cols;
      g.tiles_c[j] = (int32_t)tiles_c;
      g.row_base[j + 1] = g.row_base[j] + tiles * B;
      wgs += (tiles * B * (B / 4) + f4_per_wg - 1) / f4_per_wg;
      if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
      g.wg_base[j + 1] = (int32_t)wgs;
    }
    if (wgs > 0) {
      if (to_stack)
        hipLaunchKernelGGL(tile_copy_kernel<true>, dim3((unsigned)wgs), dim3(256), 0, stream, g, B, stack);
      else
        hipLaunchKernelGGL(tile_copy_kernel<false>, dim3((unsigned)wgs), dim3(256), 0, stream, g, B, stack);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    stack += g.row_base[g.n] * B;
  }
  return hipSuccess;
}

}  // namespace dash
