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
#include <type_traits>

#include "dash_internal.hpp"
#include "gemm_common.hpp"

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

// Element e of the start pool drawn from `seed` when the caller passes none: three SplitMix64 outputs
// (Steele, Lea and Flood, 2014: output n of the stream started at `seed` is mix(seed + n * gamma)),
// n = 3e + 1 .. 3e + 3, keep their top 22 bits; the value is (u0 + u1 + u2 - 1.5 * 2^22) * 2^-22, a
// centred sum of three uniforms.  Every step is exact in integers and fp32, so the host's copy of the
// generator gives the same bits.
__device__ __forceinline__ float pool_value(uint64_t seed, int64_t e) {
  const uint64_t gamma = 0x9E3779B97F4A7C15ull;
  uint32_t sum = 0;
  for (int q = 1; q <= 3; ++q) {
    uint64_t z = seed + (uint64_t)(3 * e + q) * gamma;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    sum += (uint32_t)(z >> 42);
  }
  return ((float)sum - 6291456.0f) * 0x1p-22f;
}

__device__ __forceinline__ float pool_at(const float* V0, uint64_t seed, int64_t e) {
  return V0 ? V0[e] : pool_value(seed, e);
}

__global__ void start_pool_kernel(uint64_t seed, int64_t n, float* V0) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) V0[e] = pool_value(seed, e);
}

// Start vectors: V0p[B, KV] = V0[:, j] / ||V0[:, j]|| for j < k, zero columns after (so every step
// reads a [B, KV] iterate with 16-byte loads); V0 null: the pool drawn from seed.  One workgroup: 32
// threads per column reduce in double, then all threads write the normalised copy.
__global__ __launch_bounds__(1024) void v0_prepare_kernel(const float* V0, uint64_t seed, int B, int k, float* V0p,
                                                          bool transposed) {
  const int j = threadIdx.x % KV, part = threadIdx.x / KV;
  __shared__ double sq[32][KV];
  __shared__ float inv[KV];
  double acc = 0.0;
  if (j < k)
    for (int i = part; i < B; i += 32) {
      const double v = pool_at(V0, seed, (int64_t)i * k + j);
      acc += v * v;
    }
  sq[part][j] = acc;
  __syncthreads();
  if (threadIdx.x < KV) {
    double t = 0.0;
    for (int q = 0; q < 32; ++q) t += sq[q][threadIdx.x];
    inv[threadIdx.x] = threadIdx.x < k ? (float)(1.0 / sqrt(t)) : 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < B * KV; e += 1024) {
    const int i = transposed ? e % B : e / KV, jj = transposed ? e / B : e % KV;
    V0p[e] = jj < k ? pool_at(V0, seed, (int64_t)i * k + jj) * inv[jj] : 0.f;
  }
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
  const float* Vsrc;    // [*, B, KV] iterate: block stride vstride (0: the prepared start vectors)
  int64_t vstride;
  const float* part_in; // partials of the previous step [N, RB, 3, KV], or null on the first step
  float* W;             // [N, B, KV]
  float* part_out;      // [N, RB, 3, KV]
  int B, k, RB;         // RB = row blocks per block
  // shifted step: W = sigma_b V - A V with sigma_b = shift_mul * shift_s[b] (shift_s null: W = A V)
  const float* shift_s;
  float shift_mul;
};

// inverse norm of column j of the current V for block b (the start vectors come normalised)
template <typename TI>
__device__ __forceinline__ float col_inv_norm(const PowerStepArgs<TI>& a, int64_t b, int j) {
  if (j >= a.k) return 0.f;
  if (!a.part_in) return 1.f;
  const float* p = a.part_in + b * (int64_t)a.RB * 3 * KV;
  double ww = 0.0;
  for (int rb = 0; rb < a.RB; ++rb) ww += p[rb * 3 * KV + j];
  return (float)(1.0 / sqrt(ww));
}

template <int V>
using IC = std::integral_constant<int, V>;

// Column partial sums (w.w, v.w, v.v) of this workgroup's rows of W = A V, and the W rows
// themselves.  acc: the wave's 32 x 32 MFMA tile (rows wave*32.., column li); vm: the iterate V
// (normalised, as the product used it) at the same 16 elements, captured from LDS when the k-loop
// staged the wave's own rows.
template <int WAVES>
__device__ __forceinline__ void power_epilogue(const float (&vm)[16], float* W, float* part_out, const f32x16& acc,
                                               int r0, int wave, int lane, float (*red)[3][KV], float sigma) {
  const int li = lane & 31, h = lane >> 5, j = li;
  float ww = 0.f, vw = 0.f, vv = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = r0 + wave * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    const float w = sigma != 0.f ? fmaf(sigma, vm[r], -acc[r]) : acc[r];
    W[(int64_t)i * KV + j] = w;
    const float v = vm[r];
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
  const int tid = wave * 64 + lane;
  if (tid < 3 * KV) {
    const int q = tid / KV, jj = tid % KV;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[w][q][jj];
    part_out[q * KV + jj] = t;
  }
}

// One power step W = A_b V_b (fp32 operands).  WAVES waves, each 32 rows x 32 columns; the
// workgroup covers RT = 32 * WAVES rows of block b and streams them in k-slices of BK = 32.
// Slices are loaded DEPTH slices ahead into a register ring (DEPTH divides B / BK), so up to
// DEPTH * 16 KiB of A per workgroup is in flight while the MFMAs run on the slice in LDS.  Three
// workgroups per CU (the register bound keeps the 4-deep ring within 168 registers): +1.5 % over two.
template <int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES, 3) void power_step_f32(PowerStepArgs<float> a) {
  constexpr int NT = 64 * WAVES;
  constexpr int RT = 32 * WAVES, BK = 32, LDA = BK + 4, LDV = KV + 4;
  constexpr int NLA = RT * BK / 4 / NT;  // float4 loads of the A slice per thread (4)
  constexpr int NLV = BK * KV / 4 / NT;  // float4 loads of the V slice per thread (1 or 2)
  __shared__ __attribute__((aligned(16))) float As[2][RT * LDA];
  __shared__ __attribute__((aligned(16))) float Vs[2][BK * LDV];
  __shared__ float inv_s[KV];
  __shared__ float red[WAVES][3][KV];
  // the RB row panels of one block share its iterate V: keep them on one XCD (one L2) by taking
  // the XCD-contiguous logical id of the product kernels
  const int64_t lid = gemm::xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = lid / a.RB;
  const int rb = (int)(lid - b * a.RB);
  const int r0 = rb * RT;
  const int B = a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const float* A = a.A + b * (int64_t)B * B;
  const float* V = a.Vsrc + b * a.vstride;
  if (tid < KV) inv_s[tid] = col_inv_norm(a, b, tid);

  f32x4 ra[DEPTH][NLA], rv[DEPTH][NLV];
  auto gload = [&](auto slot_c, int k0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + NT * r;
      const int row = f / (BK / 4), c4 = f % (BK / 4);
      ra[slot][r] = *(const f32x4*)(A + (int64_t)(r0 + row) * B + k0 + 4 * c4);
    }
#pragma unroll
    for (int r = 0; r < NLV; ++r) {
      const int f = tid + NT * r;
      const int kr = f / (KV / 4), c4 = f % (KV / 4);
      rv[slot][r] = *(const f32x4*)(V + (int64_t)(k0 + kr) * KV + 4 * c4);
    }
  };
  auto sstore = [&](auto slot_c, int buf) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + NT * r;
      const int row = f / (BK / 4), c4 = f % (BK / 4);
      *(f32x4*)&As[buf][row * LDA + 4 * c4] = ra[slot][r];
    }
#pragma unroll
    for (int r = 0; r < NLV; ++r) {
      const int f = tid + NT * r;
      const int kr = f / (KV / 4), c4 = f % (KV / 4);
      f32x4 v = rv[slot][r];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= inv_s[4 * c4 + e];
      *(f32x4*)&Vs[buf][kr * LDV + 4 * c4] = v;
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  float vm[16];  // V at the wave's own 16 accumulator elements, for the epilogue
  auto compute = [&](int kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f32x4 av = *(const f32x4*)&As[buf][(wave * 32 + li) * LDA + h * 16 + 4 * s4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float bv = Vs[buf][(h * 16 + 4 * s4 + q) * LDV + li];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q], bv, acc, 0, 0, 0);
      }
    }
    if (kt * BK == r0 + wave * 32) {  // this slice's V rows are the wave's own rows
#pragma unroll
      for (int r = 0; r < 16; ++r) vm[r] = li < a.k ? Vs[buf][(8 * (r >> 2) + 4 * h + (r & 3)) * LDV + li] : 0.f;
    }
  };
  const int KT = B / BK;
  auto step = [&](auto slot_c, int kt) {
    constexpr int slot = decltype(slot_c)::value;
    gload(slot_c, (kt + DEPTH) * BK);  // slot held slice kt, already in LDS
    compute(kt);
    sstore(IC<(slot + 1) % DEPTH>{}, (kt + 1) & 1);
    __syncthreads();
  };
  auto tail_step = [&](auto slot_c, int kt, bool store_next) {
    constexpr int slot = decltype(slot_c)::value;
    compute(kt);
    if (store_next) sstore(IC<(slot + 1) % DEPTH>{}, (kt + 1) & 1);
    __syncthreads();
  };
  gload(IC<0>{}, 0);
  if constexpr (DEPTH > 1) gload(IC<1>{}, BK);
  if constexpr (DEPTH > 2) {
    gload(IC<2>{}, 2 * BK);
    gload(IC<3>{}, 3 * BK);
  }
  __syncthreads();  // inv_s
  sstore(IC<0>{}, 0);
  __syncthreads();
  int kt = 0;
  // steady state: DEPTH divides KT, so the loop and the tail cover every slice exactly once
  for (; kt + DEPTH < KT; kt += DEPTH) {
    step(IC<0>{}, kt);
    if constexpr (DEPTH > 1) step(IC<1>{}, kt + 1);
    if constexpr (DEPTH > 2) {
      step(IC<2>{}, kt + 2);
      step(IC<3>{}, kt + 3);
    }
  }
  if constexpr (DEPTH == 1) {
    tail_step(IC<0>{}, kt, false);
  } else if constexpr (DEPTH == 2) {
    tail_step(IC<0>{}, kt, true);
    tail_step(IC<1>{}, kt + 1, false);
  } else {
    tail_step(IC<0>{}, kt, true);
    tail_step(IC<1>{}, kt + 1, true);
    tail_step(IC<2>{}, kt + 2, true);
    tail_step(IC<3>{}, kt + 3, false);
  }
  const float sigma = a.shift_s ? a.shift_mul * a.shift_s[b] : 0.f;
  power_epilogue<WAVES>(vm, a.W + b * (int64_t)B * KV, a.part_out + (b * a.RB + rb) * 3 * KV, acc, r0, wave,
                        lane, red, sigma);
}

// Streaming fp32 step for symmetric blocks, B % 128 == 0.  Since A_b is symmetric, W = A_b V is also
// A_b^T V: output row i is the sum over k of row k of A_b (at column i) times row k of V.  A
// workgroup of WPG waves covers output rows [i0, i0 + 128 WPG) of one block (the whole block when
// B <= 1024) and walks k over all B rows of A, so for every k the waves together read one
// contiguous stretch of row k (4 KiB at B = 1024) instead of 128-byte pieces of 128 rows.  Lane
// (li, h) of a wave takes A[k][iw + 4 li .. 4 li + 3] (one 16-byte load straight into registers, no
// LDS, no barrier) as the fp32 MFMA's left operand of four 32-row tiles, tile t's row m being output
// row iw + 4 m + t, and V[k][li] as the right operand, with k = kb + 8 h + p in the MFMA's slot p of
// the 16-row block kb (any pairing of rows to slots serves, as long as both operands agree).  The
// iterates are stored transposed, Vt[j][i] per block: a lane's right operands for one k-block are
// 8 consecutive floats of its column (two 16-byte loads), and its four tiles' outputs at one
// accumulator position are four consecutive rows of one column (one 16-byte store).  Each wave's
// 128 rows are one row block of the partial sums (RB = B / 128), reduced in the wave.
// SPLIT: the same operands feed the 32x32x16 bfloat16 MFMA instead: a lane's eight rows kb + 8 h + p
// of one column are exactly its eight k of that MFMA's left operand (and its eight consecutive
// iterate values its right operand), each fp32 value cut into three bfloat16 pieces (x0 = bf16(x),
// x1 = bf16(x - x0), x2 = bf16(x - x0 - x1), an exact cut), and the product is the sum of the six
// piece products with i + j <= 2, each exact in fp32 before it is accumulated: fp32 products at 6/16
// of the fp32 MFMA time, so the step is left bound by its loads.  The pieces take the step to 148
// registers, more than four waves per SIMD allow (128); this form runs two.
__device__ __forceinline__ void cut3(float x, gemm::bf16x8& p0, gemm::bf16x8& p1, gemm::bf16x8& p2, int i) {
  const __bf16 x0 = (__bf16)x;
  const float r1 = x - (float)x0;
  const __bf16 x1 = (__bf16)r1;
  p0[i] = x0;
  p1[i] = x1;
  p2[i] = (__bf16)(r1 - (float)x1);
}

template <bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(SPLIT ? 2 : 4, SPLIT ? 2 : 4))) void
power_step_stream(PowerStepArgs<float> a) {
  constexpr int D = 8;  // MFMA slots per k-block of 16 rows
  const int B = a.B;
  const int wpg = (int)(blockDim.x >> 6);
  const int gpb = B / (128 * wpg);  // workgroups per block
  const int64_t lid = gemm::xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = lid / gpb;
  const int g = (int)(lid - b * gpb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 31, h = lane >> 5;
  const int rb = g * wpg + wave;
  const int iw = rb * 128;
  const float* A = a.A + b * (int64_t)B * B;
  const float* Vt = a.Vsrc + b * a.vstride;  // [KV][B]
  const float inv = col_inv_norm(a, b, li);  // normalisation of column li (0 beyond k)
  const float* ap = A + (int64_t)(8 * h) * B + iw + 4 * li;  // + (kb + p) B
  const float* vp = Vt + (int64_t)li * B + 8 * h;              // + kb: slots 0..7 of the lane's half
  const int KB = B / 16;  // k-blocks of 16 rows; even, since B % 128 == 0
  f32x4 ra[D];
  f32x4 vb[2][2];  // right operands of k-blocks kb (vb[kb & 1]) and kb + 1: two 16-byte pieces each
#pragma unroll
  for (int p = 0; p < D; ++p) {
    ra[p] = *(const f32x4*)(ap + (int64_t)p * B);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    vb[q][0] = *(const f32x4*)(vp + 16 * q);
    vb[q][1] = *(const f32x4*)(vp + 16 * q + 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  // one k-block: each A slot is reloaded (with the next block's row) right after the MFMAs that
  // consumed it, then the block's right operands with those of the block after next; the scheduling
  // barriers keep the compiler from gathering the loads, and the two right-operand buffers alternate
  // by position (no register copies, which would wait for the loads)
  auto block = [&](int kb, auto q_c, bool reload_a, bool reload_v) {
    constexpr int q = decltype(q_c)::value;
    if constexpr (SPLIT) {
      gemm::bf16x8 b0, b1, b2;
#pragma unroll
      for (int p = 0; p < D; ++p) cut3(vb[q][p >> 2][p & 3] * inv, b0, b1, b2, p);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        gemm::bf16x8 a0, a1, a2;
#pragma unroll
        for (int p = 0; p < D; ++p) cut3(ra[p][t], a0, a1, a2, p);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b2, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b0, acc[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < D; ++p)
        if (reload_a) ra[p] = *(const f32x4*)(ap + (int64_t)(16 * (kb + 1) + p) * B);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int p = 0; p < D; ++p) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ra[p][t], vb[q][p >> 2][p & 3] * inv, acc[t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (reload_a) ra[p] = *(const f32x4*)(ap + (int64_t)(16 * (kb + 1) + p) * B);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (reload_v) {
      vb[q][0] = *(const f32x4*)(vp + 16 * (kb + 2));
      vb[q][1] = *(const f32x4*)(vp + 16 * (kb + 2) + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int kb = 0;
  for (; kb + 2 < KB; kb += 2) {
    block(kb, IC<0>{}, true, true);
    block(kb + 1, IC<1>{}, true, true);
  }
  block(kb, IC<0>{}, true, false);
  block(kb + 1, IC<1>{}, false, false);
  // epilogue: W rows (transposed store), and the column partial sums (w.w, v.w, v.v) of the wave's
  // 128 rows
  const float sigma = a.shift_s ? a.shift_mul * a.shift_s[b] : 0.f;
  float* Wt = a.W + b * (int64_t)B * KV + (int64_t)li * B;
  const float* vcol = Vt + (int64_t)li * B;
  float ww = 0.f, vw = 0.f, vv = 0.f;
  // two halves of eight rows of tiles: all loads of a half issued before its stores (the stores
  // could alias them)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
  f32x4 v4s[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int r = 8 * half + rr;
    v4s[rr] = *(const f32x4*)(vcol + iw + 4 * (8 * (r >> 2) + 4 * h + (r & 3)));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int r = 8 * half + rr;
    const int i = iw + 4 * (8 * (r >> 2) + 4 * h + (r & 3));  // rows i .. i + 3 are the four tiles
    const f32x4 v4 = v4s[rr];
    f32x4 w4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float v = v4[t] * inv;
      const float w = sigma != 0.f ? fmaf(sigma, v, -acc[t][r]) : acc[t][r];
      w4[t] = w;
      ww += w * w;
      vw += v * w;
      vv += v * v;
    }
    *(f32x4*)(Wt + i) = w4;
  }
  }
  ww += __shfl_xor(ww, 32, 64);
  vw += __shfl_xor(vw, 32, 64);
  vv += __shfl_xor(vv, 32, 64);
  if (h == 0) {
    float* po = a.part_out + (b * a.RB + rb) * 3 * KV;
    po[li] = ww;
    po[KV + li] = vw;
    po[2 * KV + li] = vv;
  }
}

// Binary16 operands: A_b prescaled in binary16, V rounded to binary16 as it is staged (transposed,
// Vs[j][k]); k-slices of BK = 64; fp32 accumulation.  Same ring as the fp32 step.
template <int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES) void power_step_f16(PowerStepArgs<_Float16> a) {
  constexpr int NT = 64 * WAVES;
  constexpr int RT = 32 * WAVES, BK = 64, LDA = BK + 8, LDV = BK + 8;
  constexpr int NLA = RT * BK / 8 / NT;  // 16-byte loads of the A slice per thread (4)
  constexpr int NLV = BK * KV / 4 / NT;  // float4 loads of the V slice per thread (2 or 4)
  __shared__ __attribute__((aligned(16))) _Float16 As[2][RT * LDA];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[2][KV * LDV];
  __shared__ float inv_s[KV];
  __shared__ float red[WAVES][3][KV];
  // the RB row panels of one block share its iterate V: keep them on one XCD (one L2) by taking
  // the XCD-contiguous logical id of the product kernels
  const int64_t lid = gemm::xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = lid / a.RB;
  const int rb = (int)(lid - b * a.RB);
  const int r0 = rb * RT;
  const int B = a.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const _Float16* A = a.A + b * (int64_t)B * B;
  const float* V = a.Vsrc + b * a.vstride;
  if (tid < KV) inv_s[tid] = col_inv_norm(a, b, tid);

  f16x8 ra[DEPTH][NLA];
  f32x4 rv[DEPTH][NLV];
  auto gload = [&](auto slot_c, int k0) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + NT * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      ra[slot][r] = *(const f16x8*)(A + (int64_t)(r0 + row) * B + k0 + 8 * c8);
    }
#pragma unroll
    for (int r = 0; r < NLV; ++r) {
      const int f = tid + NT * r;
      const int kr = f / (KV / 4), c4 = f % (KV / 4);
      rv[slot][r] = *(const f32x4*)(V + (int64_t)(k0 + kr) * KV + 4 * c4);
    }
  };
  auto sstore = [&](auto slot_c, int buf) {
    constexpr int slot = decltype(slot_c)::value;
#pragma unroll
    for (int r = 0; r < NLA; ++r) {
      const int f = tid + NT * r;
      const int row = f / (BK / 8), c8 = f % (BK / 8);
      *(f16x8*)&As[buf][row * LDA + 8 * c8] = ra[slot][r];
    }
#pragma unroll
    for (int r = 0; r < NLV; ++r) {
      const int f = tid + NT * r;
      const int kr = f / (KV / 4), c4 = f % (KV / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) Vs[buf][(4 * c4 + e) * LDV + kr] = (_Float16)(rv[slot][r][e] * inv_s[4 * c4 + e]);
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  float vm[16];  // V (binary16, as the product used it) at the wave's own 16 accumulator elements
  auto compute = [&](int kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 av = *(const f16x8*)&As[buf][(wave * 32 + li) * LDA + h * 32 + 8 * s];
      const f16x8 bv = *(const f16x8*)&Vs[buf][li * LDV + h * 32 + 8 * s];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc, 0, 0, 0);
    }
    const int off = r0 + wave * 32 - kt * BK;  // the wave's own rows within this slice, if there
    if ((unsigned)off < (unsigned)BK) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        vm[r] = li < a.k ? (float)Vs[buf][li * LDV + off + 8 * (r >> 2) + 4 * h + (r & 3)] : 0.f;
    }
  };
  const int KT = B / BK;
  auto step = [&](auto slot_c, int kt) {
    constexpr int slot = decltype(slot_c)::value;
    gload(slot_c, (kt + DEPTH) * BK);
    compute(kt);
    sstore(IC<(slot + 1) % DEPTH>{}, (kt + 1) & 1);
    __syncthreads();
  };
  auto tail_step = [&](auto slot_c, int kt, bool store_next) {
    constexpr int slot = decltype(slot_c)::value;
    compute(kt);
    if (store_next) sstore(IC<(slot + 1) % DEPTH>{}, (kt + 1) & 1);
    __syncthreads();
  };
  gload(IC<0>{}, 0);
  if constexpr (DEPTH > 1) gload(IC<1>{}, BK);
  if constexpr (DEPTH > 2) {
    gload(IC<2>{}, 2 * BK);
    gload(IC<3>{}, 3 * BK);
  }
  __syncthreads();  // inv_s
  sstore(IC<0>{}, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + DEPTH < KT; kt += DEPTH) {
    step(IC<0>{}, kt);
    if constexpr (DEPTH > 1) step(IC<1>{}, kt + 1);
    if constexpr (DEPTH > 2) {
      step(IC<2>{}, kt + 2);
      step(IC<3>{}, kt + 3);
    }
  }
  if constexpr (DEPTH == 1) {
    tail_step(IC<0>{}, kt, false);
  } else if constexpr (DEPTH == 2) {
    tail_step(IC<0>{}, kt, true);
    tail_step(IC<1>{}, kt + 1, false);
  } else {
    tail_step(IC<0>{}, kt, true);
    tail_step(IC<1>{}, kt + 1, true);
    tail_step(IC<2>{}, kt + 2, true);
    tail_step(IC<3>{}, kt + 3, false);
  }
  const float sigma = a.shift_s ? a.shift_mul * a.shift_s[b] : 0.f;
  power_epilogue<WAVES>(vm, a.W + b * (int64_t)B * KV, a.part_out + (b * a.RB + rb) * 3 * KV, acc, r0, wave,
                        lane, red, sigma);
}

// s_b = scale_b * max_{j<k} (v.w / v.v) from the last step's partials; for a shifted iteration
// (shift_s set) s_b = sigma_b - max_j (v.w / v.v)
__global__ void power_finish_kernel(const float* part, int64_t N, int RB, int k, const float* coef, float* s,
                                    const float* shift_s, float shift_mul) {
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
    const float out = shift_s ? shift_mul * shift_s[b] - mu : mu * scale;
    s[b] = any_nan ? __builtin_nanf("") : out;
  }
}

// r_b = sqrt(mean_{j<k} sum_i (W[i][j] - V0p[i][j])^2): 256 threads, column j = tid % 32, rows
// tid / 32 + 8 t, reduced in double.
__global__ __launch_bounds__(256) void probe_finish_kernel(const float* W, const float* V0p, int B, int k, float* r) {
  const int64_t b = blockIdx.x;
  const int j = threadIdx.x % KV, part = threadIdx.x / KV;
  const float* w = W + b * (int64_t)B * KV;
  double acc = 0.0;
  if (j < k)
    for (int i = part; i < B; i += 256 / KV) {
      const double e = (double)w[(int64_t)i * KV + j] - (double)V0p[(int64_t)i * KV + j];
      acc += e * e;
    }
  __shared__ double red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int q = 0; q < 256; ++q) t += red[q];
    r[b] = (float)sqrt(t / k);
  }
}

}  // namespace

size_t power_workspace_bytes(int64_t N, int B, dash_prec prec) {
  const int RB = B / 64;  // upper bound on row blocks per block
  size_t bytes = 0;
  bytes += 2 * align_up((size_t)N * B * KV * sizeof(float), 256);
  bytes += 2 * align_up((size_t)N * RB * 3 * KV * sizeof(float), 256);
  bytes += align_up((size_t)B * KV * sizeof(float), 256);       // prepared start vectors
  bytes += align_up((size_t)N * COEF_STRIDE * sizeof(float), 256);
  if (prec == DASH_FP16) bytes += align_up((size_t)N * B * B * sizeof(_Float16), 256);
  return bytes;
}

hipError_t launch_start_pool(uint64_t seed, int64_t n, float* V0, hipStream_t stream) {
  if (n < 1 || n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(start_pool_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, seed, n, V0);
  return hipGetLastError();
}

hipError_t launch_frobenius(const float* A, int64_t N, int B, float* s, hipStream_t stream) {
  if (N > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(frobenius_kernel, dim3((unsigned)N), dim3(1024), 0, stream, A, B, s);
  return hipGetLastError();
}

// Ring depth for a k-loop of KT slices: the largest of 4, 2, 1 that divides KT and is <= max_depth.
// (binary16 steps run best at 2: the 4-deep ring costs them a wave per SIMD.)
inline int ring_depth(int KT, int max_depth) {
  return (max_depth >= 4 && KT % 4 == 0) ? 4 : (KT % 2 == 0 ? 2 : 1);
}

template <typename TI, int WAVES, int DEPTH>
void launch_step(dim3 grid, hipStream_t stream, const PowerStepArgs<TI>& a) {
  if constexpr (sizeof(TI) == 4)
    hipLaunchKernelGGL((power_step_f32<WAVES, DEPTH>), grid, dim3(64 * WAVES), 0, stream, a);
  else
    hipLaunchKernelGGL((power_step_f16<WAVES, DEPTH>), grid, dim3(64 * WAVES), 0, stream, a);
}

template <typename TI, int WAVES>
void launch_step_depth(int depth, dim3 grid, hipStream_t stream, const PowerStepArgs<TI>& a) {
  if (depth == 4)
    launch_step<TI, WAVES, 4>(grid, stream, a);
  else if (depth == 2)
    launch_step<TI, WAVES, 2>(grid, stream, a);
  else
    launch_step<TI, WAVES, 1>(grid, stream, a);
}

hipError_t launch_half_prescale(const float* A, int64_t N, int B, float* coef, hipStream_t stream) {
  if (N < 1 || N > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(half_prescale_kernel, dim3((unsigned)N), dim3(256), 0, stream, A, N, B, coef);
  return hipGetLastError();
}

hipError_t launch_power_iteration(const PowerPlan& p, hipStream_t stream) {
  const bool wide = (p.B % 128 == 0);
  const int RT = wide ? 128 : 64;
  const int RB = p.B / RT;
  const int64_t grid = p.N * RB;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t err;
  // fp32 on 128-row blocks: the streaming step (row k of the symmetric block read whole), whose
  // iterates are stored transposed, [KV][B] per block
  const bool stream_f32 = p.prec != DASH_FP16 && wide;
  const bool split = p.prec == DASH_FP32_SPLIT && wide;
  hipLaunchKernelGGL(v0_prepare_kernel, dim3(1), dim3(1024), 0, stream, p.V0, p.seed, p.B, p.k, p.V0p, stream_f32);
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
  // fp32 slices are 32 wide, binary16 slices 64 wide
  const int depth = p.prec != DASH_FP16 ? ring_depth(p.B / 32, 4) : ring_depth(p.B / 64, 2);
  // waves per workgroup: the largest of 8, 4, 2, 1 dividing the block's 128-row blocks
  const int rbs = p.B / 128;
  const int wpg = !stream_f32 ? 1 : rbs % 8 == 0 ? 8 : rbs % 4 == 0 ? 4 : rbs % 2 == 0 ? 2 : 1;
  const int64_t sgrid = stream_f32 ? p.N * (p.B / (128 * wpg)) : 0;
  if (sgrid > 0x7fffffffLL) return hipErrorInvalidValue;
  for (int t = 0; t < p.steps; ++t) {
    const int cur = t & 1;
    auto fill = [&](auto& a) {
      a.Vsrc = t == 0 ? p.V0p : p.W[cur ^ 1];
      a.vstride = t == 0 ? 0 : (int64_t)p.B * KV;
      a.part_in = t == 0 ? nullptr : p.part[cur ^ 1];
      a.W = p.W[cur];
      a.part_out = p.part[cur];
      a.B = p.B;
      a.k = p.k;
      a.RB = RB;
      a.shift_s = p.shift_s;
      a.shift_mul = p.shift_mul;
    };
    if (stream_f32) {
      PowerStepArgs<float> a;
      a.A = p.A;
      fill(a);
      if (split)
        hipLaunchKernelGGL(power_step_stream<true>, dim3((unsigned)sgrid), dim3(64 * wpg), 0, stream, a);
      else
        hipLaunchKernelGGL(power_step_stream<false>, dim3((unsigned)sgrid), dim3(64 * wpg), 0, stream, a);
    } else if (p.prec != DASH_FP16) {
      PowerStepArgs<float> a;
      a.A = p.A;
      fill(a);
      launch_step_depth<float, 2>(depth, dim3((unsigned)grid), stream, a);
    } else {
      PowerStepArgs<_Float16> a;
      a.A = p.Ah;
      fill(a);
      if (wide)
        launch_step_depth<_Float16, 4>(depth, dim3((unsigned)grid), stream, a);
      else
        launch_step_depth<_Float16, 2>(depth, dim3((unsigned)grid), stream, a);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(power_finish_kernel, dim3((unsigned)p.N), dim3(64), 0, stream, p.part[(p.steps - 1) & 1], p.N,
                     RB, p.k, coef, p.s, p.shift_s, p.shift_mul);
  return hipGetLastError();
}

// Residual probe: W1 = A V, W_{t+1} = X W_t (t = 1 .. 4), unnormalised (no partials are read), then
// r_b^2 = mean_{j<k} ||W5_j - v_j||^2 with v_j the normalised start vectors.
hipError_t launch_residual_probe(const ProbePlan& p, hipStream_t stream) {
  const bool wide = (p.B % 128 == 0);
  const int RT = wide ? 128 : 64;
  const int RB = p.B / RT;
  const int64_t grid = p.N * RB;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t err;
  hipLaunchKernelGGL(v0_prepare_kernel, dim3(1), dim3(1024), 0, stream, p.V0, p.seed, p.B, p.k, p.V0p, false);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int depth = ring_depth(p.B / 32, 4);
  for (int t = 0; t < 5; ++t) {
    PowerStepArgs<float> a;
    a.A = t == 0 ? p.A : p.X;
    a.Vsrc = t == 0 ? p.V0p : p.W[(t - 1) & 1];
    a.vstride = t == 0 ? 0 : (int64_t)p.B * KV;
    a.part_in = nullptr;  // every pass multiplies the previous result as it is
    a.W = p.W[t & 1];
    a.part_out = p.part[t & 1];
    a.B = p.B;
    a.k = p.k;
    a.RB = RB;
    a.shift_s = nullptr;
    a.shift_mul = 0.f;
    if (wide)
      launch_step_depth<float, 4>(depth, dim3((unsigned)grid), stream, a);
    else
      launch_step_depth<float, 2>(depth, dim3((unsigned)grid), stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(probe_finish_kernel, dim3((unsigned)p.N), dim3(256), 0, stream, p.W[0], p.V0p, p.B, p.k, p.r);
  return hipGetLastError();
}

}  // namespace dash
