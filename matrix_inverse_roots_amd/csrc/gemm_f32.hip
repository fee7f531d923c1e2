// gemm_f32.hip -- batched fp32 B x B products on the 32x32x2 fp32 MFMA.
//
// Workgroup = 4 waves (256 threads), macro tile TILE x TILE (128, or 64 when B is not a multiple
// of 128), wave tile (TILE/2)^2, k-step 32, LDS double buffer fed from two register slots, so the
// next two k-slices are in flight while one is multiplied.  Within one k-step, lane half h of an
// MFMA takes k = h*16 + s at step s, so each lane reads 16 consecutive k of its X row with 128-bit
// LDS loads; the Y operand is a single float per lane read straight from a row of the Y tile.
// The statistics products read one operand transposed while staging it (TX / TY).  Products with
// a symmetric result (statistics, Clenshaw) compute only upper-triangle tiles (SYM) and mirror
// them: a lane's 4 consecutive accumulator rows of one column are a 16-byte piece of a mirror row,
// which the lane stores itself.
// CY: the epilogue's C operand is the right operand Y itself (Clenshaw's b_{k+1}), so the C tile
// rows [i0, i0 + TILE) pass through LDS as k-slices of Y; each wave adds (beta/alpha) C to its
// accumulators from those slices and the epilogue reads no C from memory.  MAPY: the right operand
// is staged as a Y + g I with a per-block a (Clenshaw's first b, formed inside the product).
#include <hip/hip_runtime.h>

#include "gemm_common.hpp"

namespace dash {
namespace gemm {
namespace {

template <int TILE, int TX, int TY, bool SYM, typename TO, bool CHECKS, bool CY, bool MAPY = false, bool FRZ = false>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BK = 32;
  constexpr int WT = TILE / 2;
  constexpr int MT = WT / 32;
  constexpr int LDA = BK + 4;    // As[m][k]
  constexpr int LDB = TILE + 4;  // Bs[k][n]
  constexpr int NL = TILE * BK / 4 / 256;
  constexpr int SMEM_BYTES = (2 * TILE * LDA + 2 * BK * LDB) * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  float(*As)[TILE * LDA] = reinterpret_cast<float(*)[TILE * LDA]>(smem);
  float(*Bs)[BK * LDB] = reinterpret_cast<float(*)[BK * LDB]>(smem + 2 * TILE * LDA * 4);

  TileCoord tc;
  if constexpr (FRZ) {
    if (!decode_tile_interleaved(a, SYM, tc)) return;
  } else {
    tc = decode_tile(a, SYM);
  }
  Product P = tc.prob ? a.p1 : a.p0;
  const int B = a.B;
  const int64_t off = tc.b * (int64_t)B * B;
  const float* X = (const float*)P.X + off;
  const float* Y = (const float*)P.Y + off;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  if constexpr (FRZ) {  // a block that stopped iterating: pass an operand through, or write nothing
    if (P.freeze && P.freeze[tc.b]) {
      if (P.pass == 0 || P.freeze[tc.b] == 2) return;
      const float* Z = P.pass == 1 ? X : Y;
      f32x16 pz[MT][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < MT; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = i0 + wm * WT + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            pz[mt][nt][r] = Z[(int64_t)i * B + j0 + wn * WT + nt * 32 + li];
          }
      epilogue<MT, MT, WT, WT, SYM, TO, true, true, TILE, CHECKS>(a, tc, P, pz, wm, wn, lane);
      return;
    }
  }

  // two register slots: k-slices kt + 1 and kt + 2 are in flight while slice kt is in LDS
  f32x4 ra0[NL], rb0[NL], ra1[NL], rb1[NL];
  auto gload = [&](f32x4 (&ra)[NL], f32x4 (&rb)[NL], int k0) {
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
  // MAPY (Clenshaw's first product, a launch of its own): Y = A is read as b_{d-1} = a A + g I
  const float ya = MAPY ? P.map_a * coef_of(a.epi, P.map_ia, tc.b) : 0.f;
  const float yg = MAPY ? P.map_g * coef_of(a.epi, P.map_ig, tc.b) : 0.f;
  auto sstore = [&](const f32x4 (&ra)[NL], const f32x4 (&rb)[NL], int buf, int k0) {
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
        f32x4 v = rb[r];
        if constexpr (MAPY) {
          const int d = k0 + krow - (j0 + 4 * c4);  // Y[k][j] is on the diagonal when j == k
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(v[q], ya, q == d ? yg : 0.f);
        }
        *(f32x4*)&Bs[buf][krow * LDB + 4 * c4] = v;
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
  auto compute = [&](int kt) {
    const float* as = As[kt & 1];
    const float* bs = Bs[kt & 1];
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
    if constexpr (CY) {
      // this slice holds Y rows kt*BK .. kt*BK + 31, i.e. C rows of the tile when they fall in
      // [i0, i0 + TILE); BK = 32 rows are exactly one row of 32 x 32 accumulators
      const int s_rel = kt * BK - i0;
      if (s_rel >= 0 && s_rel < TILE) {
        const float fc = a.epi.c_over_a * coef_of(a.epi, a.epi.ic, tc.b);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (wm * WT + mt * 32 != s_rel) continue;
#pragma unroll
          for (int nt = 0; nt < MT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[mt][nt][r] += fc * bs[(8 * (r >> 2) + 4 * h + (r & 3)) * LDB + wn * WT + nt * 32 + li];
        }
      }
    }
  };
  // KT = B / 32 is even; each loop pass runs two k-slices, with the register slots alternating
  gload(ra0, rb0, 0);
  sstore(ra0, rb0, 0, 0);
  __syncthreads();
  gload(ra1, rb1, BK);
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    gload(ra0, rb0, (kt + 2) * BK);
    compute(kt);
    sstore(ra1, rb1, (kt + 1) & 1, (kt + 1) * BK);
    __syncthreads();
    gload(ra1, rb1, (kt + 3) * BK);
    compute(kt + 1);
    sstore(ra0, rb0, (kt + 2) & 1, (kt + 2) * BK);
    __syncthreads();
  }
  compute(kt);
  sstore(ra1, rb1, (kt + 1) & 1, (kt + 1) * BK);
  __syncthreads();
  // last k-slice: a Clenshaw launch loads its E values first, so that their latency overlaps this
  // slice's MFMAs (the mapped first product has no E)
  float ev[CY ? MT : 1][MT][16];
  if constexpr (CY && !MAPY) load_e<MT, MT, WT, WT, TILE>(a, tc, P, wm, wn, lane, ev);
  compute(kt + 1);
  __syncthreads();
  if (CY) P.C = nullptr;  // already in the accumulators
  if constexpr (CY && MAPY)
    epilogue<MT, MT, WT, WT, SYM, TO, false, false, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane);
  else if constexpr (CY)
    epilogue<MT, MT, WT, WT, SYM, TO, false, true, TILE, CHECKS, true>(a, tc, P, acc, wm, wn, lane, ev);
  else
    epilogue<MT, MT, WT, WT, SYM, TO, true, true, TILE, CHECKS>(a, tc, P, acc, wm, wn, lane);
}

template <int TILE, bool CHECKS>
hipError_t dispatch_f32(GemmArgs& a, Trans trans, bool sym, bool c_is_y, hipStream_t stream) {
  a.tdim = a.B / TILE;
  a.tiles = sym ? a.tdim * (a.tdim + 1) / 2 : a.tdim * a.tdim;
  const bool map_y = a.p0.map_y || (a.nprob > 1 && a.p1.map_y);
  if (trans == Trans::NN) {
    if (sym && c_is_y && map_y) return launch(gemm_f32_kernel<TILE, 0, 0, true, float, CHECKS, true, true>, a, stream);
    if (sym && c_is_y) return launch(gemm_f32_kernel<TILE, 0, 0, true, float, CHECKS, true>, a, stream);
    if (sym) return launch(gemm_f32_kernel<TILE, 0, 0, true, float, CHECKS, false>, a, stream);
    if (a.p0.freeze || (a.nprob > 1 && a.p1.freeze))
      return launch_interleaved(gemm_f32_kernel<TILE, 0, 0, false, float, CHECKS, false, false, true>, a, stream);
    return launch(gemm_f32_kernel<TILE, 0, 0, false, float, CHECKS, false>, a, stream);
  }
  if (!sym) return hipErrorInvalidValue;
  if (trans == Trans::NT) return launch(gemm_f32_kernel<TILE, 0, 1, true, float, CHECKS, false>, a, stream);
  return launch(gemm_f32_kernel<TILE, 1, 0, true, float, CHECKS, false>, a, stream);
}

}  // namespace

hipError_t launch_f32(GemmArgs& a, Trans trans, bool sym, hipStream_t stream) {
  const bool checks = wants_checks(a.epi);
  const bool cy = a.epi.fold_c;
  if (a.B % 128 == 0)
    return checks ? dispatch_f32<128, true>(a, trans, sym, cy, stream)
                  : dispatch_f32<128, false>(a, trans, sym, cy, stream);
  return checks ? dispatch_f32<64, true>(a, trans, sym, cy, stream) : dispatch_f32<64, false>(a, trans, sym, cy, stream);
}

}  // namespace gemm
}  // namespace dash
