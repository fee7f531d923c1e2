// evd.hip -- inverse fourth root through an eigendecomposition A = Q diag(w) Q^T of every block of
// the stack, by a two-sided block Jacobi method.
//
// The eigendecomposition is the root solver that DASH's iterations replace ([PT] Definição do
// Problema, item 2, and Resultados Experimentais: EVD-based roots are the costly baseline; [TG]
// body).  Here it is a batched GPU solver of its own:
//
// - The B columns are cut into K = B/32 blocks of 32.  A sweep runs K-1 rounds; in each round the
//   blocks are paired by the circle (round-robin) schedule, so each pair of blocks meets once per
//   sweep and the K/2 pairs of a round are disjoint.
// - Pair kernel, one workgroup per (matrix, pair): the 64 x 64 sub-problem S = A[I u J, I u J]
//   sits in LDS (in fp64) and gets one sweep of scalar cyclic Jacobi (the same circle schedule on
//   its 64 indices: 63 inner rounds of 32 disjoint rotations, each a classical rotation that zeroes
//   one off-diagonal pair; pairs with |S_pq| <= tol sqrt(S_pp S_qq) are left alone).  The
//   accumulated 64 x 64 rotation goes to the workspace transposed (R_p^T), the form the update
//   kernel reads; the rotated S goes back to A.
// - Update kernel, one workgroup per 64 x 64 output: the off-pair blocks become
//   A_pq <- R_p^T A_pq R_q (mirrored into A_qp), and the eigenvector estimate V <- V R, as
//   32x32x2 fp32 MFMA products from LDS rows along the summed index.
// - A matrix whose whole sweep needed no rotation is done: later launches return at once for it.
//   An update whose pair rotations are all the identity is skipped.
// - Binary16 first pass (optional): the update products are formed as fp32 corrections M (R - I)
//   from binary16 operands (fp32 accumulation); the refinement pass below, in fp32, must follow it.
// - A first pass that the refinement pass follows solves its pair sub-problems in fp32 (the
//   refinement pass forms H from the input again and runs fp64 ones).
// - Refinement pass (optional, driven from api.hip): V is re-orthogonalised by Newton-Schulz steps
//   (one after an fp32 first pass, two after a binary16 one), H = V^T A V is formed from the input A
//   again, and the same sweeps run on H, rotating V.
//   This discards the rounding that the first pass accumulated in the working matrix over its many
//   dense rounds, which dominates the error at high condition numbers.
// - Finally w = diag(A), Y = V diag(w^{-1/8}) and X = Y Y^T (a triangle-only NT product: X comes
//   out exactly symmetric).
#include <hip/hip_runtime.h>

#include <cmath>

#include "dash_internal.hpp"

namespace dash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int JB = 32;         // column block width
constexpr int JS = 2 * JB;     // sub-problem order: one pair of column blocks
constexpr int JP = JS + 1;     // LDS row pitch in floats (column walks hit distinct banks)
// Scalar Jacobi sweeps per visit of a sub-problem.  One sweep per visit (an inexact inner solve)
// costs about one more outer sweep than diagonalising every sub-problem fully and a quarter of the
// inner work.
constexpr int MAX_INNER = 1;
constexpr int NTH = 256;
constexpr int TV = JS * JS / 4 / NTH;            // 16-byte pieces per thread of a 64 x 64 fp32 tile
constexpr int SU = (JS / 2) * (JS / 2) / NTH;    // 2 x 2 blocks of S per thread per inner round
constexpr int QU = JS * (JS / 2) / NTH;          // (row, rotation) items of Q per thread
static_assert(TV * NTH * 4 == JS * JS && SU * NTH == (JS / 2) * (JS / 2) && QU * NTH == JS * (JS / 2),
              "the per-thread item counts must cover the tiles exactly");

// per-matrix flags: done, sweeps of this pass, rotated in sweep (parity), sweeps of earlier passes
enum { F_DONE = 0, F_SWEEPS = 1, F_ROT = 2, F_PREV = 4, F_STRIDE = 8 };  // F_ROT + (sweep & 1)

// Circle schedule of n players (n even): in round r seat 0 holds player 0 and seat x > 0 holds
// player 1 + (x - 1 + r) mod (n - 1); seat x plays seat n - 1 - x.  Rounds 0 .. n-2 pair every two
// players exactly once.
__device__ __forceinline__ int seat(int x, int r, int n) { return x == 0 ? 0 : 1 + (x - 1 + r) % (n - 1); }

// the two column blocks I < J of pair p in round r (K blocks)
__device__ __forceinline__ void pair_blocks(int p, int r, int K, int& I, int& J) {
  const int u = seat(p, r, K), v = seat(K - 1 - p, r, K);
  I = u < v ? u : v;
  J = u < v ? v : u;
}

// global index of entry x (0..63) of a pair's index set
__device__ __forceinline__ int pidx(int x, int I, int J) { return x < JB ? I * JB + x : J * JB + x - JB; }

// Workgroup w of a launch over nb matrices with `per` workgroups each.  Workgroups are dealt to the
// 8 XCDs round-robin (w % 8), so XCD x is given the matrices m = x (mod 8), each one's workgroups
// in a row: a matrix's rotations and tiles are shared through one L2.  False for the padding
// workgroups of the last group of 8 matrices.
__device__ __forceinline__ bool xcd_item(int per, int64_t nb, int64_t& m, int& item) {
  const int64_t w = blockIdx.x, x = w & 7, slot = w >> 3;
  m = 8 * (slot / per) + x;
  item = (int)(slot % per);
  return m < nb;
}

inline int64_t xcd_grid(int64_t nb, int64_t per) { return (nb + 7) / 8 * 8 * per; }

struct JacobiArgs {
  float* A;      // [N, B, B] working copy, diagonalised in place
  float* V;      // [N, B, B] accumulated rotations
  float* R;      // [N, P, JS, JS] rotations of the current round (binary16 pass: R^T in binary16)
  int32_t* rot;  // [N, P] pair p of the current round rotated something
  float* rsc;    // binary16 pass: [N, P] power-of-two scale of pair p's stored R - I
  int32_t* flags;
  const float* coef;  // binary16 pass: per-block prescale 2^-e (CO_P2) and 2^e (CO_P2INV)
  int64_t b0, nb;  // first matrix of this launch, matrices in it
  int B, K, P, round, sweep;
  int half;        // binary16 operands in the update products
  float tol;
};

// The sub-problem and its accumulated rotation live in LDS in fp64 (fp64 FMA runs at the fp32
// rate here) and are rounded to fp32 once, when written out: a rotation accumulated in fp32 over the
// thousands of plane rotations of one visit drifts from orthogonality by ~sqrt(count) ulp,
// and applying such a near-rotation to the off-pair blocks every round moves the eigenvalues.
// The binary16 pass (its products round every operand to binary16 anyway) keeps them in fp32
// (T = float): half the LDS bytes per access and twice the workgroups per compute unit.
template <typename T>
struct CS {
  T c, s;
};

// |a_pq| > tol sqrt(a_pp a_qq): the pair is rotated (fp32: the square roots taken apart, so that the
// product of two diagonal entries can neither overflow nor underflow)
__device__ __forceinline__ bool needs_rotation(double app, double aqq, double apq, double tol) {
  return fabs(apq) > tol * sqrt(fabs(app * aqq));
}
__device__ __forceinline__ bool needs_rotation(float app, float aqq, float apq, float tol) {
  return fabsf(apq) > tol * (sqrtf(fabsf(app)) * sqrtf(fabsf(aqq)));
}

template <typename T>
__global__ __launch_bounds__(NTH) void jacobi_pair_kernel(JacobiArgs a) {
  __shared__ T S[JS * JP];
  __shared__ T Q[JS * JP];
  __shared__ CS<T> rot_cs[JS / 2];  // (c, s) of rotation k
  __shared__ int2 rot_pq[JS / 2];     // its index pair p < q
  __shared__ int rotated[MAX_INNER];
  __shared__ int round_rot[2];  // inner round r rotates something (parity of r)
  int64_t m;
  int p;
  if (!xcd_item(a.P, a.nb, m, p)) return;
  const int64_t b = a.b0 + m;
  if (a.flags[b * F_STRIDE + F_DONE]) return;
  int I, J;
  pair_blocks(p, a.round, a.K, I, J);
  const int tid = threadIdx.x;
  const int B = a.B;
  float* Ab = a.A + b * (int64_t)B * B;
  {
    f32x4 v[TV];
#pragma unroll
    for (int u = 0; u < TV; ++u) {  // 16-byte pieces never straddle the two halves
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      v[u] = *(const f32x4*)(Ab + (int64_t)pidx(i, I, J) * B + pidx(4 * c4, I, J));
    }
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) S[i * JP + 4 * c4 + q] = v[u][q];
    }
  }
#pragma unroll
  for (int u = 0; u < JS * JS / NTH; ++u) {
    const int e = tid + NTH * u, i = e >> 6, j = e & 63;
    Q[i * JP + j] = i == j ? T(1) : T(0);
  }
  if (tid < MAX_INNER) rotated[tid] = 0;
  if (tid < 2) round_rot[tid] = 0;
  __syncthreads();
  const T tol = a.tol;
  for (int sw = 0; sw < MAX_INNER; ++sw) {
    for (int r = 0; r < JS - 1; ++r) {
      const int rr = sw * (JS - 1) + r;  // inner round count, for the flag parity
      if (tid < JS / 2) {
        const int u = seat(tid, r, JS), v = seat(JS - 1 - tid, r, JS);
        const int pp = u < v ? u : v, qq = u < v ? v : u;
        const T app = S[pp * JP + pp], aqq = S[qq * JP + qq], apq = S[pp * JP + qq];
        T c = 1, s = 0;
        if (needs_rotation(app, aqq, apq, tol)) {
          // the rotation that zeroes entry (pp, qq): t = tan of its angle, the smaller root of
          // t^2 + 2 theta t - 1 = 0 (a theta whose square overflows gives t = 0: no rotation)
          const T th = (aqq - app) / (T(2) * apq);
          const T t = (th >= T(0) ? T(1) : T(-1)) / (fabs(th) + sqrt(th * th + T(1)));
          c = T(1) / sqrt(t * t + T(1));
          s = t * c;
          rotated[sw] = 1;
          round_rot[rr & 1] = 1;
        }
        rot_cs[tid] = CS<T>{c, s};
        rot_pq[tid] = make_int2(pp, qq);
      }
      __syncthreads();
      // a round whose 32 rotations are all the identity changes nothing; the flag of the next
      // round was last read before the previous barrier
      const bool any = round_rot[rr & 1];
      if (tid == 0) round_rot[(rr + 1) & 1] = 0;
      // S <- J^T S J: one 2 x 2 block (rows of rotation k, columns of rotation l) per item; this
      // thread's items are l = tid % 32, k = tid / 32 + 8 u.  All loads are issued before the
      // arithmetic so that their latencies overlap.
      if (any) {
        const int l = tid & 31, kb = tid >> 5;
        const int2 pql = rot_pq[l];
        const CS<T> csl = rot_cs[l];
        int2 pqk[SU];
        CS<T> csk[SU];
        T x[SU][4];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          pqk[u] = rot_pq[kb + 8 * u];
          csk[u] = rot_cs[kb + 8 * u];
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          x[u][0] = S[pqk[u].x * JP + pql.x];
          x[u][1] = S[pqk[u].x * JP + pql.y];
          x[u][2] = S[pqk[u].y * JP + pql.x];
          x[u][3] = S[pqk[u].y * JP + pql.y];
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const T cl = csl.c, sl = csl.s, ck = csk[u].c, sk = csk[u].s;
          const T y00 = cl * x[u][0] - sl * x[u][1], y01 = sl * x[u][0] + cl * x[u][1];  // columns
          const T y10 = cl * x[u][2] - sl * x[u][3], y11 = sl * x[u][2] + cl * x[u][3];
          T z00 = ck * y00 - sk * y10, z10 = sk * y00 + ck * y10;  // rows
          T z01 = ck * y01 - sk * y11, z11 = sk * y01 + ck * y11;
          if (kb + 8 * u == l && sl != T(0)) z01 = z10 = T(0);  // the entry a rotation annihilates
          S[pqk[u].x * JP + pql.x] = z00;
          S[pqk[u].x * JP + pql.y] = z01;
          S[pqk[u].y * JP + pql.x] = z10;
          S[pqk[u].y * JP + pql.y] = z11;
        }
      }
      // Q <- Q J: items (k, i), row i = tid % 64, k = tid / 64 + 4 u
      if (any) {
        const int i = tid & 63, kb = tid >> 6;
        int2 pqk[QU];
        CS<T> csk[QU];
        T x0[QU], x1[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          pqk[u] = rot_pq[kb + 4 * u];
          csk[u] = rot_cs[kb + 4 * u];
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          x0[u] = Q[i * JP + pqk[u].x];
          x1[u] = Q[i * JP + pqk[u].y];
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          Q[i * JP + pqk[u].x] = csk[u].c * x0[u] - csk[u].s * x1[u];
          Q[i * JP + pqk[u].y] = csk[u].s * x0[u] + csk[u].c * x1[u];
        }
      }
      __syncthreads();
    }
    if (!rotated[sw]) break;
  }
  if (rotated[0]) {
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (float)S[i * JP + 4 * c4 + q];
      *(f32x4*)(Ab + (int64_t)pidx(i, I, J) * B + pidx(4 * c4, I, J)) = v;
    }
  }
  if (a.half) {
    // (R - I)^T in binary16 (the update kernel reads both of its uses row-wise), scaled by the power
    // of two 1/rsc that maps its largest entry into (1/2, 1]: entries far below binary16's normal
    // range would otherwise be lost, and with them the small rotations of a converging block
    __shared__ float wmax[NTH / 64];
    float d[TV][4];
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        d[u][q] = (float)(Q[c * JP + i] - (c == i ? T(1) : T(0)));
        mx = fmaxf(mx, fabsf(d[u][q]));
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    int ex = 0;
    if (mx > 0.f && isfinite(mx)) {
      const float mant = frexpf(mx, &ex);  // mx = mant 2^ex, mant in [1/2, 1)
      if (mant == 0.5f) --ex;
    }
    const float down = ldexpf(1.f, -ex);
    _Float16* Rh = (_Float16*)a.R + (b * a.P + p) * (int64_t)(JS * JS);
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      f16x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (_Float16)(d[u][q] * down);
      *(f16x4*)(Rh + i * JS + 4 * c4) = v;
    }
    if (tid == 0) a.rsc[b * a.P + p] = ldexpf(1.f, ex);
  } else {
    // R^T, rounded to fp32: the update kernel reads both of its uses row-wise
    float* Rb = a.R + (b * a.P + p) * (int64_t)(JS * JS);
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (float)Q[(4 * c4 + q) * JP + i];
      *(f32x4*)(Rb + i * JS + 4 * c4) = v;
    }
  }
  if (tid == 0) {
    a.rot[b * a.P + p] = rotated[0];
    if (rotated[0]) atomicOr(&a.flags[b * F_STRIDE + F_ROT + (a.sweep & 1)], 1);
  }
}

// The fp32 update products read both operands from LDS rows along the summed index k, 16 bytes at a
// time: X[i][k] for the left operand, Y^T[j][k] for the right one (the pair kernel stores R^T, and
// T = A_pq R_q is staged transposed from the accumulators).  Rows are FP = 68 floats: 16-byte reads
// stay aligned, and the 16 rows the LDS serves together start 4 banks apart, covering its 64 banks.
constexpr int FP = JS + 4;

// out = X Y^T over the 64-long index (X, Yt: 64 x 64 fp32 in LDS, pitch FP) -> the wave's 32 x 32
// quadrant, on the 32x32x2 fp32 MFMA: lane half h takes k = 32 h + 4 m + j at step (m, j), one
// 16-byte read per operand feeding four MFMAs.
__device__ __forceinline__ f32x16 mm64v(const float* X, const float* Yt, int wm, int wn, int li, int h) {
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const float* xr = X + (wm * JB + li) * FP;
  const float* yr = Yt + (wn * JB + li) * FP;
#pragma unroll
  for (int m = 0; m < JB / 4; ++m) {
    const f32x4 xa = *(const f32x4*)(xr + JB * h + 4 * m);
    const f32x4 yb = *(const f32x4*)(yr + JB * h + 4 * m);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[j], yb[j], acc, 0, 0, 0);
  }
  return acc;
}

// row of element r of this lane's accumulator in the wave's quadrant (the 32x32 MFMA layout: element
// r of lane l is row 8(r/4) + 4(l/32) + r%4, column l%32)
__device__ __forceinline__ int acc_row(int r, int wm, int h) { return wm * JB + 8 * (r >> 2) + 4 * h + (r & 3); }

// A 64 x 64 fp32 tile through registers: piece u of this thread is row e/16, columns 4(e%16) ..
// 4(e%16)+3 of the tile, e = tid + NTH u.  Row i of the tile is at src + row_off(i), its column c
// at + col(c) (a 16-byte piece never straddles the two 32-column halves of a pair's index set).
template <typename RowOff, typename Col>
__device__ __forceinline__ void fetch_tile(f32x4 (&v)[TV], const float* src, RowOff row_off, Col col, int tid) {
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
    v[u] = *(const f32x4*)(src + row_off(i) + col(4 * c4));
  }
}

// the tile (fetched by fetch_tile) into LDS rows of pitch FP
__device__ __forceinline__ void stage_tile_v(float* T, const f32x4 (&v)[TV], int tid) {
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
    *(f32x4*)&T[i * FP + 4 * c4] = v[u];
  }
}

// Items of one matrix: P(P-1)/2 off-pair blocks A_pq (p < q), then P * B/64 tiles of V (64 rows
// by one pair's 64 columns).
__global__ __launch_bounds__(NTH) void jacobi_update_kernel(JacobiArgs a) {
  __shared__ __attribute__((aligned(16))) float X[JS * FP];   // left operand, then T^T
  __shared__ __attribute__((aligned(16))) float Rq[JS * FP];  // R_q^T, then the result (pitch JP)
  __shared__ __attribute__((aligned(16))) float Rp[JS * FP];  // R_p^T
  const int P = a.P, B = a.B;
  const int PA = P * (P - 1) / 2;
  const int per = PA + P * (B / JS);
  int64_t m;
  int t;
  if (!xcd_item(per, a.nb, m, t)) return;
  const int64_t b = a.b0 + m;
  if (a.flags[b * F_STRIDE + F_DONE]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const float* Rm = a.R + b * P * (int64_t)(JS * JS);  // R^T of every pair of the round
  auto rot_row = [](int i) { return (int64_t)i * JS; };
  auto rot_col = [](int c) { return c; };
  if (t < PA) {
    int p = 0;
    while (t >= P - 1 - p) {
      t -= P - 1 - p;
      ++p;
    }
    const int q = p + 1 + t;
    if (!a.rot[b * P + p] && !a.rot[b * P + q]) return;  // R_p = R_q = I: nothing changes
    int Ip, Jp, Iq, Jq;
    pair_blocks(p, a.round, a.K, Ip, Jp);
    pair_blocks(q, a.round, a.K, Iq, Jq);
    float* Ab = a.A + b * (int64_t)B * B;
    f32x4 va[TV], vq[TV], vp[TV];
    fetch_tile(va, Ab, [&](int i) { return (int64_t)pidx(i, Ip, Jp) * B; }, [&](int c) { return pidx(c, Iq, Jq); },
               tid);
    fetch_tile(vq, Rm + q * JS * JS, rot_row, rot_col, tid);
    fetch_tile(vp, Rm + p * JS * JS, rot_row, rot_col, tid);
    stage_tile_v(X, va, tid);
    stage_tile_v(Rq, vq, tid);
    stage_tile_v(Rp, vp, tid);
    __syncthreads();
    f32x16 acc = mm64v(X, Rq, wm, wn, li, h);  // T = A_pq R_q
    __syncthreads();
    // T^T into X: element r of this lane is T[wm 32 + 8 (r/4) + 4 h + r%4][wn 32 + li], four
    // consecutive rows per group of r
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) v[q2] = acc[4 * g + q2];
      *(f32x4*)&X[(wn * JB + li) * FP + wm * JB + 8 * g + 4 * h] = v;
    }
    __syncthreads();
    acc = mm64v(Rp, X, wm, wn, li, h);  // R_p^T T
    float* O = Rq;  // R_q^T is dead: the result, pitch JP
#pragma unroll
    for (int r = 0; r < 16; ++r) O[acc_row(r, wm, h) * JP + wn * JB + li] = acc[r];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      f32x4 v, w;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = O[i * JP + 4 * c4 + r];
        w[r] = O[(4 * c4 + r) * JP + i];
      }
      *(f32x4*)(Ab + (int64_t)pidx(i, Ip, Jp) * B + pidx(4 * c4, Iq, Jq)) = v;
      *(f32x4*)(Ab + (int64_t)pidx(i, Iq, Jq) * B + pidx(4 * c4, Ip, Jp)) = w;
    }
  } else {
    t -= PA;
    const int rb = t / P, q = t - rb * P;
    if (!a.rot[b * P + q]) return;
    int Iq, Jq;
    pair_blocks(q, a.round, a.K, Iq, Jq);
    float* Vb = a.V + b * (int64_t)B * B + (int64_t)rb * JS * B;
    f32x4 vv[TV], vq[TV];
    fetch_tile(vv, Vb, [&](int i) { return (int64_t)i * B; }, [&](int c) { return pidx(c, Iq, Jq); }, tid);
    fetch_tile(vq, Rm + q * JS * JS, rot_row, rot_col, tid);
    stage_tile_v(X, vv, tid);
    stage_tile_v(Rq, vq, tid);
    __syncthreads();
    const f32x16 acc = mm64v(X, Rq, wm, wn, li, h);  // V_tile R_q
#pragma unroll
    for (int r = 0; r < 16; ++r) Vb[(int64_t)acc_row(r, wm, h) * B + pidx(wn * JB + li, Iq, Jq)] = acc[r];
  }
}

// The binary16 update: the same items as jacobi_update_kernel, each product written as a correction
// M R = M + M (R - I) whose second term is formed on the binary16 matrix cores (32x32x16, fp32
// accumulation) from operands rounded to binary16 as they are staged, and added to the fp32 M in
// the epilogue.  The rounding error of a product is then a binary16 fraction of |M| |R - I|:
// binary16's unit roundoff while the rotations are large (the first sweeps of a dense block), less
// as they approach the identity.  It is not small enough for the refinement pass, whose rotations
// between nearly equal eigenvalues stay large while H is nearly diagonal: that pass runs in fp32.
// A_pq's operand is first scaled by the block's power-of-two 2^-e (its entries then lie within the
// largest eigenvalue times 2^-e, far inside the binary16 range); R - I is stored scaled by a power
// of two per pair (largest entry in (1/2, 1]) and the eigenvector tiles have entries in [-1, 1].  A and V stay fp32 in memory.  Operand
// tiles sit in LDS row-wise along the summed index, so each lane reads 8 consecutive binary16
// values per matrix-core step: X[i][k] for the left operand and Y^T[j][k] for the right one.
constexpr int HP = JS + 8;  // binary16 LDS pitch: 144-byte rows keep 16-byte reads aligned

// out = X Y^T over the 64-long index (X, Yt: 64 x 64 binary16 in LDS, pitch HP) -> the wave's
// 32 x 32 quadrant.  Lane half h takes k = 32 h + 8 s .. 32 h + 8 s + 7 at step s: both operands use
// the same k order, so the sum is over every k once.
__device__ __forceinline__ f32x16 mm64h(const _Float16* X, const _Float16* Yt, int wm, int wn, int li, int h) {
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < JS / 16; ++s) {
    const f16x8 xa = *(const f16x8*)&X[(wm * JB + li) * HP + JB * h + 8 * s];
    const f16x8 yb = *(const f16x8*)&Yt[(wn * JB + li) * HP + JB * h + 8 * s];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa, yb, acc, 0, 0, 0);
  }
  return acc;
}

// a 64 x 64 fp32 tile (fetched by fetch_tile) times c, rounded to binary16 into LDS (pitch HP)
__device__ __forceinline__ void stage_tile_h(_Float16* T, const f32x4 (&v)[TV], float c, int tid) {
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
    f16x4 hv;
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = (_Float16)(v[u][q] * c);
    *(f16x4*)&T[i * HP + 4 * c4] = hv;
  }
}

constexpr int HV = JS * JS / 8 / NTH;  // 16-byte pieces per thread of a 64 x 64 binary16 tile

// a 64 x 64 binary16 tile (row pitch JS in memory) through registers into LDS (pitch HP)
__device__ __forceinline__ void fetch_rot_h(f16x8 (&v)[HV], const _Float16* src, int tid) {
#pragma unroll
  for (int u = 0; u < HV; ++u) {
    const int e = tid + NTH * u, i = e >> 3, c8 = e & 7;
    v[u] = *(const f16x8*)(src + i * JS + 8 * c8);
  }
}

__device__ __forceinline__ void stage_rot_h(_Float16* T, const f16x8 (&v)[HV], int tid) {
#pragma unroll
  for (int u = 0; u < HV; ++u) {
    const int e = tid + NTH * u, i = e >> 3, c8 = e & 7;
    *(f16x8*)&T[i * HP + 8 * c8] = v[u];
  }
}

// the fp32 tile (fetched by fetch_tile) into LDS with pitch JP
__device__ __forceinline__ void stage_tile_f(float* T, const f32x4 (&v)[TV], int tid) {
#pragma unroll
  for (int u = 0; u < TV; ++u) {
    const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) T[i * JP + 4 * c4 + q] = v[u][q];
  }
}

__global__ __launch_bounds__(NTH) void jacobi_update_h_kernel(JacobiArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 X[JS * HP];   // left operand, then T^T
  __shared__ __attribute__((aligned(16))) _Float16 Rq[JS * HP];  // (R_q - I)^T
  __shared__ __attribute__((aligned(16))) _Float16 Rp[JS * HP];  // (R_p - I)^T
  __shared__ float O[JS * JP];                                   // the fp32 input, then the result
  const int P = a.P, B = a.B;
  const int PA = P * (P - 1) / 2;
  const int per = PA + P * (B / JS);
  int64_t m;
  int t;
  if (!xcd_item(per, a.nb, m, t)) return;
  const int64_t b = a.b0 + m;
  if (a.flags[b * F_STRIDE + F_DONE]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const _Float16* Rh = (const _Float16*)a.R + b * P * (int64_t)(JS * JS);
  if (t < PA) {
    int p = 0;
    while (t >= P - 1 - p) {
      t -= P - 1 - p;
      ++p;
    }
    const int q = p + 1 + t;
    if (!a.rot[b * P + p] && !a.rot[b * P + q]) return;
    int Ip, Jp, Iq, Jq;
    pair_blocks(p, a.round, a.K, Ip, Jp);
    pair_blocks(q, a.round, a.K, Iq, Jq);
    float* Ab = a.A + b * (int64_t)B * B;
    const float p2 = a.coef[b * COEF_STRIDE + CO_P2], p2inv = a.coef[b * COEF_STRIDE + CO_P2INV];
    const float uq = p2inv * a.rsc[b * P + q], up = p2inv * a.rsc[b * P + p];  // powers of two
    f32x4 va[TV];
    f16x8 vq[HV], vp[HV];
    fetch_tile(va, Ab, [&](int i) { return (int64_t)pidx(i, Ip, Jp) * B; }, [&](int c) { return pidx(c, Iq, Jq); },
               tid);
    fetch_rot_h(vq, Rh + q * JS * JS, tid);
    fetch_rot_h(vp, Rh + p * JS * JS, tid);
    stage_tile_h(X, va, p2, tid);
    stage_tile_f(O, va, tid);
    stage_rot_h(Rq, vq, tid);
    stage_rot_h(Rp, vp, tid);
    __syncthreads();
    f32x16 acc = mm64h(X, Rq, wm, wn, li, h);  // 2^-e A_pq (R_q - I) / rsc_q
    float tv[16];                               // T = A_pq R_q at this lane's elements
#pragma unroll
    for (int r = 0; r < 16; ++r) tv[r] = O[acc_row(r, wm, h) * JP + wn * JB + li] + acc[r] * uq;
    __syncthreads();
    // (2^-e T)^T into X: element r of this lane is T[wm 32 + 8 (r/4) + 4 h + r%4][wn 32 + li], four
    // rows in a row per group of r
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f16x4 hv;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) hv[q2] = (_Float16)(tv[4 * g + q2] * p2);
      *(f16x4*)&X[(wn * JB + li) * HP + wm * JB + 8 * g + 4 * h] = hv;
    }
    __syncthreads();
    acc = mm64h(Rp, X, wm, wn, li, h);  // 2^-e (R_p - I)^T T / rsc_p
#pragma unroll
    for (int r = 0; r < 16; ++r) O[acc_row(r, wm, h) * JP + wn * JB + li] = tv[r] + acc[r] * up;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + NTH * u, i = e >> 4, c4 = e & 15;
      f32x4 v, w;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = O[i * JP + 4 * c4 + r];
        w[r] = O[(4 * c4 + r) * JP + i];
      }
      *(f32x4*)(Ab + (int64_t)pidx(i, Ip, Jp) * B + pidx(4 * c4, Iq, Jq)) = v;
      *(f32x4*)(Ab + (int64_t)pidx(i, Iq, Jq) * B + pidx(4 * c4, Ip, Jp)) = w;
    }
  } else {
    t -= PA;
    const int rb = t / P, q = t - rb * P;
    if (!a.rot[b * P + q]) return;
    int Iq, Jq;
    pair_blocks(q, a.round, a.K, Iq, Jq);
    float* Vb = a.V + b * (int64_t)B * B + (int64_t)rb * JS * B;
    f32x4 vv[TV];
    f16x8 vq[HV];
    fetch_tile(vv, Vb, [&](int i) { return (int64_t)i * B; }, [&](int c) { return pidx(c, Iq, Jq); }, tid);
    fetch_rot_h(vq, Rh + q * JS * JS, tid);
    stage_tile_h(X, vv, 1.f, tid);
    stage_tile_f(O, vv, tid);
    stage_rot_h(Rq, vq, tid);
    __syncthreads();
    const f32x16 acc = mm64h(X, Rq, wm, wn, li, h);  // V_tile (R_q - I)
    const float uq = a.rsc[b * P + q];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = acc_row(r, wm, h);
      Vb[(int64_t)i * B + pidx(wn * JB + li, Iq, Jq)] = O[i * JP + wn * JB + li] + acc[r] * uq;
    }
  }
}

// Sweep bookkeeping, one thread per matrix.  sweep == 0: start of a pass (the first pass clears
// the count of earlier sweeps, a later one adds the previous pass's sweeps to it).  sweep t >= 1
// (sweep t-1 has completed): a matrix whose sweep t-1 rotated nothing is done; F_SWEEPS counts the
// sweeps run in this pass.
__global__ void jacobi_sweep_kernel(int32_t* flags, int64_t N, int sweep, int pass) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= N) return;
  int32_t* f = flags + b * F_STRIDE;
  if (sweep == 0) {
    f[F_PREV] = pass == 0 ? 0 : f[F_PREV] + f[F_SWEEPS];
    f[F_DONE] = 0;
    f[F_SWEEPS] = 0;
    f[F_ROT] = 0;
    f[F_ROT + 1] = 0;
    return;
  }
  if (!f[F_DONE]) {
    f[F_SWEEPS] = sweep;
    if (!f[F_ROT + ((sweep - 1) & 1)]) f[F_DONE] = 1;
  }
  f[F_ROT + (sweep & 1)] = 0;
}

// V <- I for every matrix
__global__ void identity_kernel(float* V, int64_t N, int B) {
  const int64_t n4 = N * (int64_t)B * B / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t idx = 4 * e;
    const int64_t in = idx % ((int64_t)B * B);
    const int i = (int)(in / B), j0 = (int)(in % B);
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (i == j0 + q) ? 1.f : 0.f;
    *(f32x4*)(V + idx) = v;
  }
}

// Per matrix: eigenvalues w_j = A_jj, column scales w_j^{-1/8} (NaN for a w_j that is not finite or
// not > 0, status bit 0), eigenvalue and sweep outputs, status bit 2 when not converged.
__global__ __launch_bounds__(256) void evd_finish_kernel(const float* A, int64_t b0, int B, const int32_t* flags,
                                                         float* scale, float* eigvals, int32_t* sweeps,
                                                         int32_t* status) {
  const int64_t b = b0 + blockIdx.x;
  const float* Ab = A + b * (int64_t)B * B;
  int bad = 0;
  for (int j = threadIdx.x; j < B; j += blockDim.x) {
    const float w = Ab[(int64_t)j * B + j];
    const bool ok = w > 0.f && isfinite(w);
    bad |= !ok;
    // w^{-1/8} as three square roots (each exactly equivariant under w -> 4^k w)
    scale[b * B + j] = ok ? (float)(1.0 / sqrt(sqrt(sqrt((double)w)))) : __builtin_nanf("");
    if (eigvals) eigvals[b * B + j] = w;
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    const int32_t* f = flags + b * F_STRIDE;
    if (sweeps) sweeps[b] = f[F_PREV] + f[F_SWEEPS];
    if (status) status[b] |= (bad ? 1 : 0) | (f[F_DONE] ? 0 : 4);
  }
}

// Y[b][i][j] = V[b][i][j] * scale[b][j]  (Y may be V)
__global__ void column_scale_kernel(const float* V, const float* scale, float* Y, int64_t N, int B) {
  const int64_t n4 = N * (int64_t)B * B / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t idx = 4 * e;
    const int64_t b = idx / ((int64_t)B * B);
    const int j0 = (int)(idx % B);
    const f32x4 v = *(const f32x4*)(V + idx);
    const f32x4 s = *(const f32x4*)(scale + b * B + j0);
    *(f32x4*)(Y + idx) = v * s;
  }
}

unsigned stream_grid(int64_t n4) {
  const int64_t g = (n4 + 255) / 256;
  return (unsigned)(g < 16384 ? g : 16384);
}

}  // namespace

size_t evd_workspace_bytes(int64_t N, int B) {
  size_t bytes = 2 * align_up((size_t)N * B * B * sizeof(float), 256);       // V, T
  bytes += align_up((size_t)N * (B / JS) * JS * JS * sizeof(float), 256);    // R
  bytes += align_up((size_t)N * (B / JS) * sizeof(int32_t), 256);            // pair flags
  bytes += align_up((size_t)N * B * sizeof(float), 256);                     // column scales
  bytes += align_up((size_t)N * F_STRIDE * sizeof(int32_t), 256);            // flags
  bytes += align_up((size_t)N * COEF_STRIDE * sizeof(float), 256);           // binary16 prescale
  bytes += align_up((size_t)N * (B / JS) * sizeof(float), 256);              // binary16 R - I scales
  return bytes;
}

hipError_t launch_identity(float* V, int64_t N, int B, hipStream_t stream) {
  hipLaunchKernelGGL(identity_kernel, dim3(stream_grid(N * (int64_t)B * B / 4)), dim3(256), 0, stream, V, N, B);
  return hipGetLastError();
}

hipError_t launch_jacobi(const JacobiPlan& p, hipStream_t stream) {
  const int B = p.B;
  const int K = B / JB, P = B / JS;
  const int64_t N = p.N;
  hipError_t err;
  const unsigned fgrid = (unsigned)((N + 255) / 256);
  JacobiArgs a;
  a.A = p.A;
  a.V = p.V;
  a.R = p.R;
  a.rot = p.rot;
  a.rsc = p.rsc;
  a.flags = p.flags;
  a.B = B;
  a.K = K;
  a.P = P;
  a.tol = p.tol;
  a.half = p.half ? 1 : 0;
  a.coef = p.coef;
  if (p.half && (!p.coef || !p.rsc)) return hipErrorInvalidValue;
  // matrices per launch, so that a grid stays below 2^32 work-items
  const int64_t max_wg = 0xffffffffLL / NTH;
  const int64_t per_update = (int64_t)P * (P - 1) / 2 + (int64_t)P * (B / JS);
  const int64_t chunk = max_wg / per_update / 8 * 8;
  for (int t = 0; t <= p.max_sweeps; ++t) {
    hipLaunchKernelGGL(jacobi_sweep_kernel, dim3(fgrid), dim3(256), 0, stream, p.flags, N, t, p.pass);
    if (t == p.max_sweeps) break;
    a.sweep = t;
    for (int r = 0; r < K - 1; ++r) {
      a.round = r;
      for (int64_t b0 = 0; b0 < N; b0 += chunk) {
        const int64_t nb = N - b0 < chunk ? N - b0 : chunk;
        a.b0 = b0;
        a.nb = nb;
        if (p.pair_f32)
          hipLaunchKernelGGL(jacobi_pair_kernel<float>, dim3((unsigned)xcd_grid(nb, P)), dim3(NTH), 0, stream, a);
        else
          hipLaunchKernelGGL(jacobi_pair_kernel<double>, dim3((unsigned)xcd_grid(nb, P)), dim3(NTH), 0, stream, a);
        if (p.half)
          hipLaunchKernelGGL(jacobi_update_h_kernel, dim3((unsigned)xcd_grid(nb, per_update)), dim3(NTH), 0, stream,
                             a);
        else
          hipLaunchKernelGGL(jacobi_update_kernel, dim3((unsigned)xcd_grid(nb, per_update)), dim3(NTH), 0, stream, a);
      }
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // the sweep kernel of t == max_sweeps closed the pass (done flag, sweep count)
  return hipGetLastError();
}

hipError_t launch_evd_finish(const EvdFinish& f, hipStream_t stream) {
  const int64_t max_wg = 0xffffffffLL / 256;
  for (int64_t b0 = 0; b0 < f.N; b0 += max_wg) {
    const int64_t nb = f.N - b0 < max_wg ? f.N - b0 : max_wg;
    hipLaunchKernelGGL(evd_finish_kernel, dim3((unsigned)nb), dim3(256), 0, stream, f.A, b0, f.B, f.flags, f.scale,
                       f.eigvals, f.sweeps, f.status);
  }
  hipLaunchKernelGGL(column_scale_kernel, dim3(stream_grid(f.N * (int64_t)f.B * f.B / 4)), dim3(256), 0, stream, f.V,
                     f.scale, f.Y, f.N, f.B);
  return hipGetLastError();
}

}  // namespace dash
