// scale.hip -- per-block spectral scale estimates.
//
// Frobenius: s_i = ||A_i||_F, one streaming pass ([PT] Definição do Problema, item 3).
//
// Multi-Power-Iteration ([PT] Metodologia, item 2, "Multi-Power-Iteration"; [TG] body, Rayleigh
// quotient): k <= 32 start vectors per block advance together, so one step is the skinny product
// W = A_i V (B x B times B x 32) -- a stream over A_i with 16 flop per fp32 byte, run on the 32x32
// MFMA with the V slice staged in LDS.  Each workgroup owns 128 (or 64) rows of one block and
// writes, besides its rows of W, the column partial sums (w.w, v.w, v.v) of those rows; the next
// step reduces the partials of its block to normalise V on the fly while loading it, and the last
// step's partials give the Rayleigh quotients mu_j = v.w / v.v and s_i = max_j mu_j.  No atomics:
// the result is deterministic.
//
// Binary16 variant ([PT] Principais Contribuições, item 4: half-precision power iteration): A_i is
// cast once to binary16 after a power-of-two prescale 2^-e, e = ceil(log2 max_j A_i[j][j]), so its
// entries stay below 1 in magnitude; V is rounded to binary16 as it is staged; accumulation is fp32.
#include <hip/hip_runtime.h>

#include <cmath>

#include "dash_internal.hpp"

namespace dash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int KV = 32;  // columns of the power-iteration iterate (k <= 32, unused columns are zero)

// ------------------------------------------------------------------------------------------------
// Frobenius norm: one 1024-thread workgroup per block.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void frobenius_kernel(const float* A, int B, float* s) {
  const int64_t b = blockIdx.x;
  const f32x4* p = (const f32x4*)(A + b * (int64_t)B * B);
  const int64_t n4 = (int64_t)B * B / 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = threadIdx.x; i < n4; i += 4 * 1024) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t idx = i + u * 1024;
      if (idx < n4) {
        const f32x4 v = p[idx];
        acc[u] += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      }
    }
  }
  double t = (double)acc[0] + (double)acc[1] + (double)acc[2] + (double)acc[3];
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
  __shared__ double red[16];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < 16; ++w) tot += red[w];
    s[b] = (float)sqrt(tot);
  }
}

// ------------------------------------------------------------------------------------------------
// Power iteration
// ------------------------------------------------------------------------------------------------

// inverse column norms of the shared start vectors V0[B, k]; zero for padding columns j >= k
__global__ void v0_inverse_norms_kernel(const float* V0, int B, int k, float* inv) {
  const int j = threadIdx.x;
  if (j >= KV) return;
  if (j >= k) {
    inv[j] = 0.f;
    return;
  }
  double acc = 0.0;
  for (int i = 0; i < B; ++i) {
    const double v = V0[(int64_t)i * k + j];
    acc += v * v;
  }
  inv[j] = (float)(1.0 / sqrt(acc));
}

// binary16 prescale per block: coef[P2] = 2^-e, coef[P2INV] = 2^e, e = ceil(log2 max diag)
__global__ void half_prescale_kernel(const float* A, int64_t N, int B, float* coef) {
  const int64_t b = blockIdx.x;
  const float* a = A + b * (int64_t)B * B;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < B; i += blockDim.x) m = fmaxf(m, a[(int64_t)i * B + i]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float dmax = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) dmax = fmaxf(dmax, red[w]);
    float* c = coef + b * COEF_STRIDE;
    if (!(dmax > 0.f) || !isfinite(dmax)) {
      c[CO_P2] = 0.f;
      c[CO_P2INV] = 0.f;
      return;
    }
    int ex;
    const float mant = frexpf(dmax, &ex);  // dmax = mant * 2^ex, mant in [0.5, 1)
    const int e = (mant == 0.5f) ? ex - 1 : ex;
    c[CO_P2] = ldexpf(1.f, -e);
    c[CO_P2INV] = ldexpf(1.f, e);
  }
}

template <typename TI>
struct PowerStepArgs {
  const TI* A;          // [N, B, B]
  const float* Vsrc;    // [*, B, vld]: block stride vstride (0: shared start vectors)
  int64_t vstride;
  int vld;
  const float* v0inv;   // inverse norms of the shared start vectors (first step), or null
  const float* part_in; // partials of the previous step [N, RB, 3, KV] (later steps)
  float* W;             // [N, B, KV]
  float* part_out;      // [N, RB, 3, KV]
  int B, k, RB;         // RB = row blocks per block
};

// inverse norm of column j of the current V for block b
template <typename TI>
__device__ __forceinline__ float col_inv_norm(const PowerStepArgs<TI>& a, int64_t b, int j) {
  if (j >= a.k) return 0.f;
  if (a.v0inv) return a.v0inv[j];
  const float* p = a.part_in + b * (int64_t)a.RB * 3 * KV;
  double ww = 0.0;
  for (int rb = 0; rb < a.RB; ++rb) ww += p[rb * 3 * KV + j];
  return (float)(1.0 / sqrt(ww));
}

template <typename TI>
__device__ __forceinline__ float stage_v(float v) {
  return (float)(TI)v;  // binary16 rounding of the iterate when TI is _Float16
}

// WAVES waves, each 32 rows x 32 columns; the workgroup covers RT = 32 * WAVES rows of block b.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void power_step_f32(PowerStepArgs<float> a) {
  constexpr int RT = 32 * WAVES, BK = 32, LDA = BK + 4, LDV = KV + 4;
  __shared__ __attribute__((aligned(16))) float As[2][RT * LDA];
  __shared__ __attribute__((aligned(16))) float Vs[2][BK * LDV];
  __shared__ float inv_s[KV];
  __shared__ float red[WAVES][3][KV];
  const int64_t b = blockIdx.x / a.RB;
  const int rb = (int)(blockIdx.x - b * a.RB);
  const int r0 = rb * RT;
  const int B = a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const float* A = a.A + b * (int64_t)B * B;
  const float* V = a.Vsrc + b * a.vstride;
  if (tid < KV) inv_s[tid] = col_inv_norm(a, b, tid);
  __syncthreads();

  constexpr int NLA = RT * BK / 4 / (64 * WAVES);  // float4 loads of the A slice per thread (= 4)
  f32x4 ra[NLA];
  float rv[BK * KV / (64 * WAVES)];
  constexpr int NV = BK * KV / (64 * WAVES);
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int row = f / (BK / 4), c4 = f % (BK / 4);
      ra[r] = *(const f32x4*)(A + (int64_t)(r0 + row) * B + k0 + 4 * c4);
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int kr = f / KV, j = f % KV;
      rv[r] = (j < a.k) ? V[(int64_t)(k0 + kr) * a.vld + j] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int row = f / (BK / 4), c4 = f % (BK / 4);
      *(f32x4*)&As[buf][row * LDA + 4 * c4] = ra[r];
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int kr = f / KV, j = f % KV;
      Vs[buf][kr * LDV + j] = rv[r] * inv_s[j];
    }
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int KT = B / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f32x4 av = *(const f32x4*)&As[buf][(wave * 32 + li) * LDA + h * 16 + 4 * s4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float bv = Vs[buf][(h * 16 + 4 * s4 + q) * LDV + li];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q], bv, acc, 0, 0, 0);
      }
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: W rows, column partial sums of this workgroup's rows
  const int j = li;
  const float invj = inv_s[j];
  float ww = 0.f, vw = 0.f, vv = 0.f;
  float* Wb = a.W + b * (int64_t)B * KV;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = r0 + wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    const float w = acc[r];
    Wb[(int64_t)i * KV + j] = w;
    const float v = (j < a.k) ? V[(int64_t)i * a.vld + j] * invj : 0.f;
    ww += w * w;
    vw += v * w;
    vv += v * v;
  }
  ww += __shfl_xor(ww, 32, 64);
  vw += __shfl_xor(vw, 32, 64);
  vv += __shfl_xor(vv, 32, 64);
  if (h == 0) {
    red[wave][0][j] = ww;
    red[wave][1][j] = vw;
    red[wave][2][j] = vv;
  }
  __syncthreads();
  if (tid < 3 * KV) {
    const int q = tid / KV, jj = tid % KV;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[w][q][jj];
    a.part_out[(b * a.RB + rb) * 3 * KV + q * KV + jj] = t;
  }
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void power_step_f16(PowerStepArgs<_Float16> a) {
  constexpr int RT = 32 * WAVES, BK = 64, LDA = BK + 8, LDV = BK + 8;
  __shared__ __attribute__((aligned(16))) _Float16 As[2][RT * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[2][KV * LDV];  // transposed: Vs[j][k]
  __shared__ float inv_s[KV];
  __shared__ float red[WAVES][3][KV];
  const int64_t b = blockIdx.x / a.RB;
  const int rb = (int)(blockIdx.x - b * a.RB);
  const int r0 = rb * RT;
  const int B = a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const _Float16* A = a.A + b * (int64_t)B * B;
  const float* V = a.Vsrc + b * a.vstride;
  if (tid < KV) inv_s[tid] = col_inv_norm(a, b, tid);
  __syncthreads();

  constexpr int NLA = RT * BK / 8 / (64 * WAVES);  // 16-byte loads of the A slice per thread (= 4)
  constexpr int NV = BK * KV / (64 * WAVES);
  f16x8 ra[NLA];
  float rv[NV];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      ra[r] = *(const f16x8*)(A + (int64_t)(r0 + row) * B + k0 + 8 * c8);
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int kr = f / KV, j = f % KV;
      rv[r] = (j < a.k) ? V[(int64_t)(k0 + kr) * a.vld + j] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      *(f16x8*)&As[buf][row * LDA + 8 * c8] = ra[r];
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int f = tid + 64 * WAVES * r;
      const int kr = f / KV, j = f % KV;
      Vs[buf][j * LDV + kr] = (_Float16)(rv[r] * inv_s[j]);
    }
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int KT = B / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 av = *(const f16x8*)&As[buf][(wave * 32 + li) * LDA + h * 32 + 8 * s];
      const f16x8 bv = *(const f16x8*)&Vs[buf][li * LDV + h * 32 + 8 * s];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  const int j = li;
  const float invj = inv_s[j];
  float ww = 0.f, vw = 0.f, vv = 0.f;
  float* Wb = a.W + b * (int64_t)B * KV;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = r0 + wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    const float w = acc[r];
    Wb[(int64_t)i * KV + j] = w;
    const float v = (j < a.k) ? stage_v<_Float16>(V[(int64_t)i * a.vld + j] * invj) : 0.f;
    ww += w * w;
    vw += v * w;
    vv += v * v;
  }
  ww += __shfl_xor(ww, 32, 64);
  vw += __shfl_xor(vw, 32, 64);
  vv += __shfl_xor(vv, 32, 64);
  if (h == 0) {
    red[wave][0][j] = ww;
    red[wave][1][j] = vw;
    red[wave][2][j] = vv;
  }
  __syncthreads();
  if (tid < 3 * KV) {
    const int q = tid / KV, jj = tid % KV;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[w][q][jj];
    a.part_out[(b * a.RB + rb) * 3 * KV + q * KV + jj] = t;
  }
}

// s_b = scale_b * max_{j<k} (v.w / v.v) from the last step's partials
__global__ void power_finish_kernel(const float* part, int64_t N, int RB, int k, const float* coef, float* s) {
  const int64_t b = blockIdx.x;
  const int j = threadIdx.x;
  float mu = -INFINITY;
  if (j < k) {
    double vw = 0.0, vv = 0.0;
    const float* p = part + b * (int64_t)RB * 3 * KV;
    for (int rb = 0; rb < RB; ++rb) {
      vw += p[rb * 3 * KV + KV + j];
      vv += p[rb * 3 * KV + 2 * KV + j];
    }
    mu = (float)(vw / vv);
    if (mu != mu) mu = __builtin_nanf("");
  }
  // max over the wave; a NaN quotient propagates so that the block is flagged by the solver
  bool any_nan = (j < k) && (mu != mu);
  for (int o = 32; o > 0; o >>= 1) {
    mu = fmaxf(mu, __shfl_xor(mu, o, 64));
    any_nan |= (bool)__shfl_xor((int)any_nan, o, 64);
  }
  if (j == 0) {
    const float scale = coef ? coef[b * COEF_STRIDE + CO_P2INV] : 1.f;
    s[b] = any_nan ? __builtin_nanf("") : mu * scale;
  }
}

}  // namespace

size_t power_workspace_bytes(int64_t N, int B, dash_prec prec) {
  const int RB = B / 64;  // upper bound on row blocks per block
  size_t bytes = 0;
  bytes += 2 * align_up((size_t)N * B * KV * sizeof(float), 256);
  bytes += 2 * align_up((size_t)N * RB * 3 * KV * sizeof(float), 256);
  bytes += 256;                                                  // v0 inverse norms
  bytes += align_up((size_t)N * COEF_STRIDE * sizeof(float), 256);
  if (prec == DASH_FP16) bytes += align_up((size_t)N * B * B * sizeof(_Float16), 256);
  return bytes;
}

hipError_t launch_frobenius(const float* A, int64_t N, int B, float* s, hipStream_t stream) {
  if (N > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(frobenius_kernel, dim3((unsigned)N), dim3(1024), 0, stream, A, B, s);
  return hipGetLastError();
}

hipError_t launch_power_iteration(const PowerPlan& p, hipStream_t stream) {
  const bool wide = (p.B % 128 == 0);
  const int RT = wide ? 128 : 64;
  const int RB = p.B / RT;
  const int64_t grid = p.N * RB;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t err;
  hipLaunchKernelGGL(v0_inverse_norms_kernel, dim3(1), dim3(64), 0, stream, p.V0, p.B, p.k, p.v0inv);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const float* coef = nullptr;
  if (p.prec == DASH_FP16) {
    hipLaunchKernelGGL(half_prescale_kernel, dim3((unsigned)p.N), dim3(256), 0, stream, p.A, p.N, p.B, p.coef);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    Affine cast;
    cast.X = p.A;
    cast.D = p.Ah;
    cast.d_prec = DASH_FP16;
    cast.a = 1.f;
    cast.ia = CO_P2;
    cast.coef = p.coef;
    if ((err = launch_affine(cast, p.N, p.B, stream)) != hipSuccess) return err;
    coef = p.coef;
  }
  for (int t = 0; t < p.steps; ++t) {
    const int cur = t & 1;
    if (p.prec == DASH_FP32) {
      PowerStepArgs<float> a;
      a.A = p.A;
      a.Vsrc = t == 0 ? p.V0 : p.W[cur ^ 1];
      a.vstride = t == 0 ? 0 : (int64_t)p.B * KV;
      a.vld = t == 0 ? p.k : KV;
      a.v0inv = t == 0 ? p.v0inv : nullptr;
      a.part_in = t == 0 ? nullptr : p.part[cur ^ 1];
      a.W = p.W[cur];
      a.part_out = p.part[cur];
      a.B = p.B;
      a.k = p.k;
      a.RB = RB;
      if (wide)
        hipLaunchKernelGGL(power_step_f32<4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(power_step_f32<2>, dim3((unsigned)grid), dim3(128), 0, stream, a);
    } else {
      PowerStepArgs<_Float16> a;
      a.A = p.Ah;
      a.Vsrc = t == 0 ? p.V0 : p.W[cur ^ 1];
      a.vstride = t == 0 ? 0 : (int64_t)p.B * KV;
      a.vld = t == 0 ? p.k : KV;
      a.v0inv = t == 0 ? p.v0inv : nullptr;
      a.part_in = t == 0 ? nullptr : p.part[cur ^ 1];
      a.W = p.W[cur];
      a.part_out = p.part[cur];
      a.B = p.B;
      a.k = p.k;
      a.RB = RB;
      if (wide)
        hipLaunchKernelGGL(power_step_f16<4>, dim3((unsigned)grid), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(power_step_f16<2>, dim3((unsigned)grid), dim3(128), 0, stream, a);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(power_finish_kernel, dim3((unsigned)p.N), dim3(64), 0, stream, p.part[(p.steps - 1) & 1], p.N,
                     RB, p.k, coef, p.s);
  return hipGetLastError();
}

}  // namespace dash
