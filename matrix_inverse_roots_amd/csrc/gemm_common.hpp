// gemm_common.hpp -- pieces shared by the batched-product kernels (gemm_f32.hip, gemm_f16.hip,
// gemm_split.hip):
// launch arguments, the XCD-aware workgroup -> (problem, block, tile) map and the fused epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include "dash_internal.hpp"

namespace dash {
namespace gemm {


typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The 2-byte operand formats of the half-precision products: binary16 (_Float16) and bfloat16
// (__bf16).  Both multiply on the 32x32x16 MFMA with fp32 accumulation; v8 is the operand of one
// lane (8 consecutive k), v4 four consecutive elements of a row.
template <typename TE>
struct Half;
template <>
struct Half<_Float16> {
  typedef f16x8 v8;
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Half<__bf16> {
  typedef bf16x8 v8;
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct GemmArgs {
  Product p0, p1;
  int nprob;
  int64_t N;
  int B;
  int tiles;  // tiles per product (all tiles, or the upper triangle when sym)
  int tdim;   // B / TILE
  Epilogue epi;
};

// the monitor / status code of the epilogues is compiled only into the launches that ask for it
inline bool wants_checks(const Epilogue& e) { return e.monitor || e.status; }

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

// (row, column) of tile t of a block: all tiles row by row, or the upper triangle row by row (sym)
__device__ __forceinline__ void tile_rc(const GemmArgs& a, bool sym, int t, int& ti, int& tj) {
  if (sym) {
    int r = 0;
    while (t >= a.tdim - r) {
      t -= a.tdim - r;
      ++r;
    }
    ti = r;
    tj = r + t;
  } else {
    ti = t / a.tdim;
    tj = t - ti * a.tdim;
  }
}

__device__ __forceinline__ TileCoord decode_tile(const GemmArgs& a, bool sym) {
  const int64_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t per_prob = a.N * a.tiles;
  TileCoord c;
  c.prob = (int)(lid / per_prob);
  const int64_t rem = lid - (int64_t)c.prob * per_prob;
  c.b = rem / a.tiles;
  tile_rc(a, sym, (int)(rem - c.b * a.tiles), c.ti, c.tj);
  return c;
}

// Block-interleaved variant for launches whose blocks carry unequal work (some blocks of an adaptive
// solve have stopped): XCD x takes the blocks b = x (mod 8), each with all of its (problem, tile)
// items in a row, so stopped and running blocks spread evenly over the XCDs whatever their order
// in the stack.  The grid is padded to a multiple of 8 blocks (launch_interleaved); false for the
// padding.
__device__ __forceinline__ bool decode_tile_interleaved(const GemmArgs& a, bool sym, TileCoord& c) {
  const int64_t w = blockIdx.x, x = w & 7, slot = w >> 3;
  const int64_t per_block = (int64_t)a.nprob * a.tiles;
  c.b = 8 * (slot / per_block) + x;
  const int item = (int)(slot % per_block);
  c.prob = item / a.tiles;
  tile_rc(a, sym, item - c.prob * a.tiles, c.ti, c.tj);
  return c.b < a.N;
}

// Operand map of the half-precision products: the 8 consecutive elements Z[row][col0 .. col0 + 7]
// of a staged chunk become a Z + g I.  a is a power of two (the callers' -1/4 and -1/2), so a z is
// exact unless it is subnormal, and the diagonal element a z + g (g = 5/4 or 3/2, exact in both
// formats) is rounded once (an exact a z below the half-ulp of g cannot move the rounding): each
// result equals the exact value rounded to the operand format once, as an fp32 elementwise pass
// that stores that format would give.  Only chunks that hold a diagonal element take the branch.
template <typename TE>
__device__ __forceinline__ typename Half<TE>::v8 operand_map(typename Half<TE>::v8 v, int row, int col0, float a,
                                                             float g) {
  typename Half<TE>::v8 r = v * (TE)a;
  const int d = row - col0;
  if ((unsigned)d < 8u) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q == d) r[q] = r[q] + (TE)g;
  }
  return r;
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
// SYM (triangle-only products, no D2): only tiles ti <= tj run.  Each element is stored at (i, j),
// and at (j, i) by the same lane: its 4 consecutive r are 4 consecutive rows of one column, i.e. a
// 16-byte piece of a row of the mirror.  In a diagonal tile the direct stores keep i <= j and the
// mirror i < j, so no element is written twice.  The monitor counts off-diagonal kept elements
// twice under SYM.  C/E loads of one row of accumulators are issued before its stores (D may alias
// E: each lane reads and writes only its own elements, so loading the chunk first is still exact);
// with E_PRE, E's values come from ev_pre (load_e).
template <typename TO>
struct Vec4;
template <>
struct Vec4<float> {
  typedef float type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec4<_Float16> {
  typedef _Float16 type __attribute__((ext_vector_type(4)));
};

// E values of a lane's accumulator elements, loaded ahead of the epilogue (E_PRE) so that their
// latency overlaps the last k-slice of the product.
template <int MTM, int MTN, int WTM, int WTN, int TILE>
__device__ __forceinline__ void load_e(const GemmArgs& a, const TileCoord& tc, const Product& P, int wm, int wn,
                                       int lane, float (&ev)[MTM][MTN][16]) {
  const int B = a.B;
  const float* E = P.E + tc.b * (int64_t)B * B;
  const int li = lane & 31, h = lane >> 5;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = j0 + wn * WTN + nt * 32 + li;
        ev[mt][nt][r] = E[(int64_t)i * B + j];
      }
}

// HAS_C / HAS_E: the launch may carry C / E operands (each still optional at run time, except
// that E_PRE takes E's values from ev_pre, loaded by load_e).  HAS_D2: the launch may carry a second
// output (full products only).  AMAX: the largest |D| that the wave stored goes to *amax_out (a
// plain store by lane 0; NaN values are passed over), when amax_out is set.  MLDS (SYM, fp32
// output): the mirror goes through the wave's own MLDS_FLOATS floats of LDS at mlds, one 32 x 32
// accumulator at a time: the lane's four consecutive rows of a column are one 16-byte row piece of
// the transposed block, stored to LDS (row pitch 36 floats: the 16 lanes that the LDS serves
// together fall on distinct banks) and read back as 16-byte pieces of whole 128-byte rows, so each
// store instruction writes 8 full 128-byte rows of the mirror instead of 32-byte pieces of 32 rows.
// The wave alone reads what it wrote, so no barrier is needed; the caller's LDS must be free.
constexpr int MLDS_PITCH = 36, MLDS_FLOATS = 32 * MLDS_PITCH;
template <int MTM, int MTN, int WTM, int WTN, bool SYM, typename TO, bool HAS_C, bool HAS_E, int TILE, bool CHECKS,
          bool E_PRE = false, bool HAS_D2 = true, bool AMAX = false, bool MLDS = false>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                         const f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane,
                                         const float (*ev_pre)[MTN][16] = nullptr, float* amax_out = nullptr,
                                         float* mlds = nullptr) {
  static_assert(!MLDS || (SYM && sizeof(TO) == 4), "the LDS mirror is for fp32 triangle-only products");
  typedef typename Vec4<TO>::type v4;
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
  TO* D2 = (HAS_D2 && !SYM && P.D2) ? (TO*)P.D2 + off : nullptr;
  const float* C = P.C ? P.C + off : nullptr;
  const float* E = P.E ? P.E + off : nullptr;
  const int li = lane & 31, h = lane >> 5;
  const int i0 = tc.ti * TILE, j0 = tc.tj * TILE;
  const bool diag_tile = SYM && tc.ti == tc.tj;
  float mon = 0.f, amax = 0.f;
  bool bad = false;
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
        cv[nt][r] = (HAS_C && C) ? C[idx] : 0.f;
        if (E_PRE)
          ev[nt][r] = ev_pre[mt][nt][r];
        else
          ev[nt][r] = (HAS_E && E) ? E[idx] : 0.f;
      }
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int il0 = wm * WTM + mt * 32 + 8 * r4 + 4 * h;  // rows il0 .. il0 + 3 of the tile
        const int jl = wn * WTN + nt * 32 + li;
        v4 pk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 4 * r4 + q;
          const int il = il0 + q;
          const int i = i0 + il, j = j0 + jl;
          const float x = acc[mt][nt][r];
          float v = al * x + be * cv[nt][r] + de * ev[nt][r];
          if (i == j) v += ga;
          pk[q] = cvt_out<TO>(v);
          const int64_t idx = (int64_t)i * B + j;
          if (!diag_tile || il <= jl) {
            D[idx] = pk[q];
            if (AMAX) amax = fmaxf(amax, fabsf(v));  // (NaN leaves it unchanged)
          }
          float v2 = 0.f;
          if (D2) {
            v2 = al2 * x + (i == j ? ga2 : 0.f);
            D2[idx] = cvt_out<TO>(v2);
          }
          if (CHECKS && !(diag_tile && il > jl)) {
            bad |= !isfinite(v) || (D2 && !isfinite(v2));
            if (e.monitor) {
              const float dd = v - (i == j ? 1.f : 0.f);
              mon += (SYM && i != j) ? 2.f * dd * dd : dd * dd;
            }
          }
        }
        if (SYM && MLDS) {  // transposed block T[jl - (wn WTN + nt 32)][il - (wm WTM + mt 32)]
          *(v4*)&mlds[li * MLDS_PITCH + 8 * r4 + 4 * h] = pk;
        } else if (SYM) {
          TO* md = D + (int64_t)(j0 + jl) * B + i0 + il0;  // mirror row j, columns i .. i + 3
          if (!diag_tile || il0 + 3 < jl) {
            *(v4*)md = pk;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (il0 + q < jl) md[q] = pk[q];
          }
        }
      }
      if constexpr (SYM && MLDS) {
        // rows 8 q + lane / 8 of the transposed 32 x 32 block, 16 bytes (columns 4 (lane % 8) ..)
        // per lane; on a diagonal tile only the mirror's strict lower part (column < row)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 8 * q + (lane >> 3), cc = 4 * (lane & 7);
          const v4 t = *(const v4*)&mlds[rr * MLDS_PITCH + cc];
          const int jl = wn * WTN + nt * 32 + rr, il = wm * WTM + mt * 32 + cc;
          TO* md = D + (int64_t)(j0 + jl) * B + i0 + il;
          if (!diag_tile || il + 3 < jl) {
            *(v4*)md = t;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (il + c < jl) md[c] = t[c];
          }
        }
      }
    }
  }
  if (CHECKS && e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (CHECKS && e.status && bad) atomicOr(&e.status[b], 2);
  if (AMAX && amax_out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if (lane == 0) *amax_out = amax;
  }
}

// Word 3 of a raw buffer resource on this architecture: 32-bit data format, no swizzle, byte
// offsets (the accesses here are untyped).
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

// Epilogue of the split kernels (fp32 output; C optional when HAS_C, E optional; no second
// output): the arithmetic of `epilogue` (D = al x + be C + de E, plus ga on the diagonal), with
// every access through a buffer resource over the block, so that the lane's part of a byte offset
// is a register, the row's part a scalar and the sub-block's column a constant: a load or store
// takes no address arithmetic, and the tile's parts differ by uniform branches only.  SYM: the
// upper-triangle tile and its mirror, staged through the wave's MLDS_FLOATS floats of LDS at mlds
// as in `epilogue`; on a diagonal tile the 32 x 32 sub-blocks below the diagonal store nothing,
// those on it store their upper part (row <= column) and mirror their strict upper part, and
// those above store and mirror everything.  AMAX and CHECKS as in `epilogue`.
template <int MTM, int MTN, int WTM, int WTN, bool SYM, bool HAS_C, int TILE, bool CHECKS, bool AMAX>
__device__ __forceinline__ void epilogue_split(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                               const f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane,
                                               float* amax_out, float* mlds) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const Epilogue& e = a.epi;
  const int B = a.B;
  const int64_t b = tc.b;
  const int64_t off = b * (int64_t)B * B;
  const float al = e.alpha * coef_of(e, e.ia, b);
  const float be = e.beta * coef_of(e, e.ib, b);
  const float de = e.delta * coef_of(e, e.id, b);
  const float ga = e.gamma * coef_of(e, e.ig, b);
  auto rsrc = [&](const void* p) {  // (the block's address is the same in every lane: say so)
    const uint64_t a64 = (uint64_t)((const float*)p + off);
    const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a64 >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a64);
    return __builtin_amdgcn_make_buffer_rsrc((void*)u, (short)0, B * B * 4, BUFFER_RSRC_WORD3);
  };
  const bool has_c = HAS_C && P.C, has_e = P.E;
  const __amdgpu_buffer_rsrc_t drs = rsrc(P.D);
  const __amdgpu_buffer_rsrc_t crs = has_c ? rsrc(P.C) : drs;
  const __amdgpu_buffer_rsrc_t ers = has_e ? rsrc(P.E) : drs;
  auto ld = [&](__amdgpu_buffer_rsrc_t rs, int v, int s) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, v, s, 0));
  };
  auto st = [&](float x, int v, int s) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), drs, v, s, 0);
  };
  const int li = lane & 31, h = lane >> 5;
  const int swm = __builtin_amdgcn_readfirstlane(wm), swn = __builtin_amdgcn_readfirstlane(wn);
  const int vlane = (4 * h * B + li) * 4;                     // lane part: row 4 h, column li
  const int vmir = ((lane >> 3) * B + 4 * (lane & 7)) * 4;    // mirror: row lane / 8, column 4 (lane % 8)
  const bool diag_tile = SYM && tc.ti == tc.tj;
  float mon = 0.f, amax = 0.f;
  bool bad = false;
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt) {
      // the sub-block's tile-local origin (ib, jb) and block-level origin (row0, col0)
      const int ib = swm * WTM + mt * 32, jb = swn * WTN + nt * 32;
      if (diag_tile && ib > jb) continue;
      const int row0 = tc.ti * TILE + ib, col0 = tc.tj * TILE + jb;
      const bool on_diag = row0 == col0;  // holds the block's diagonal elements (row 4h + rr, column li)
      const bool masked = SYM && on_diag;
      float cv[16], ev[16], v[16];
      // element r: row row0 + rr(r) + 4 h, column col0 + li
      auto srow = [&](int r) { return ((row0 + 8 * (r >> 2) + (r & 3)) * B + col0) * 4; };
      if (has_c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) cv[r] = ld(crs, vlane, srow(r));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) cv[r] = 0.f;
      }
      if (has_e) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ev[r] = ld(ers, vlane, srow(r));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) ev[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 8 * (r >> 2) + (r & 3) + 4 * h;  // row within the sub-block (column li)
        float x = al * acc[mt][nt][r] + be * cv[r] + de * ev[r];
        if (on_diag && il == li) x += ga;
        v[r] = x;
        const bool keep = !masked || il <= li;
        if (masked) {
          if (keep) st(x, vlane, srow(r));
        } else {
          st(x, vlane, srow(r));
        }
        if (AMAX && keep) amax = fmaxf(amax, fabsf(x));  // (NaN leaves it unchanged)
        if (CHECKS && keep) {
          bad |= !isfinite(x);
          if (e.monitor) {
            const bool dg = on_diag && il == li;
            const float dd = x - (dg ? 1.f : 0.f);
            mon += (SYM && !dg) ? 2.f * dd * dd : dd * dd;
          }
        }
      }
      if constexpr (SYM) {
        // the transposed sub-block through LDS: the lane's four consecutive rows of column li are
        // row li of the transpose, columns 8 r4 + 4 h ..; read back as rows 8 q + lane / 8,
        // columns 4 (lane % 8) .. 4 (lane % 8) + 3, stored to row col0 + 8 q + lane / 8 of D
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4v pk;
#pragma unroll
          for (int q = 0; q < 4; ++q) pk[q] = v[4 * r4 + q];
          *(f32x4v*)&mlds[li * MLDS_PITCH + 8 * r4 + 4 * h] = pk;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = 8 * q + (lane >> 3), cc = 4 * (lane & 7);
          const f32x4v t = *(const f32x4v*)&mlds[rr * MLDS_PITCH + cc];
          const int so = ((col0 + 8 * q) * B + row0) * 4;
          if (!masked) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), drs, vmir, so, 0);
          } else {  // only the mirror's strict lower part: column cc + c < row rr
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (cc + c < rr) st(t[c], vmir + 4 * c, so);
          }
        }
      }
    }
  if (CHECKS && e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (CHECKS && e.status && bad) atomicOr(&e.status[b], 2);
  if (AMAX && amax_out) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if (lane == 0) *amax_out = amax;
  }
}

// Epilogue for binary16 outputs (no C/E operands, no second output).  Kept elements are stored
// straight from the accumulators with 2-byte stores (lanes 0-31 cover 64 contiguous bytes of a
// row).  SYM mirrors through LDS: in the 32x32 accumulator layout a lane's 4 consecutive r are 4
// consecutive rows of one column, i.e. 4 consecutive halves of a row of the transposed tile, so
// the transposed tile T[jl][il] is written with one 8-byte LDS store per 4 values and read back as
// 16-byte rows (a diagonal tile stores everything directly and the mirror then overwrites its
// strict lower part).  Monitor and status (CHECKS) as in `epilogue`.  smem: TILE * (TILE + 8)
// halves when SYM.
template <typename TE, int MTM, int MTN, int WTM, int WTN, bool SYM, int TILE, bool CHECKS>
__device__ __forceinline__ void epilogue_staged_f16(const GemmArgs& a, const TileCoord& tc, const Product& P,
                                                    const f32x16 (&acc)[MTM][MTN], int wm, int wn, int lane,
                                                    char* smem) {
  typedef typename Half<TE>::v4 h4;
  typedef typename Half<TE>::v8 h8;
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
  TE* T = (TE*)smem;
  TE* D = (TE*)P.D + off;
  float mon = 0.f;
  bool bad = false;
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int il0 = wm * WTM + mt * 32 + 8 * r4 + 4 * h;  // rows il0 .. il0 + 3
        const int jl = wn * WTN + nt * 32 + li;
        h4 pk;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int il = il0 + q;
          const bool on_diag = (i0 + il == j0 + jl);
          const float v = al * acc[mt][nt][4 * r4 + q] + (on_diag ? ga : 0.f);
          const TE hv = (TE)v;
          pk[q] = hv;
          // a diagonal tile stores its lower part too; the mirror overwrites it after the barrier
          D[(int64_t)(i0 + il) * B + j0 + jl] = hv;
          if (CHECKS && !(diag_tile && il > jl)) {
            bad |= !isfinite(v);
            if (e.monitor) {
              const float dd = v - (on_diag ? 1.f : 0.f);
              mon += (SYM && !on_diag) ? 2.f * dd * dd : dd * dd;
            }
          }
        }
        if (SYM) *(h4*)&T[jl * PITCH + il0] = pk;
      }
  if (CHECKS && e.monitor) {
    mon = wave_sum(mon);
    if (lane == 0) atomicAdd(&e.monitor[b * e.mon_stride], e.mon_mul * mon);
  }
  if (CHECKS && e.status && bad) atomicOr(&e.status[b], 2);
  if (!SYM) return;
  __syncthreads();
  const int nthreads = blockDim.x;
  for (int g = threadIdx.x; g < TILE * TILE / 8; g += nthreads) {
    const int jl = g / (TILE / 8), c8 = g - jl * (TILE / 8);
    const int il = 8 * c8;
    TE* dst = D + (int64_t)(j0 + jl) * B + i0 + il;  // mirror element (j, i) = value at (i, j)
    if (!diag_tile || il + 7 < jl) {
      *(h8*)dst = *(const h8*)&T[jl * PITCH + il];
    } else if (il < jl) {  // the chunk crossing the diagonal: strict upper part only
      for (int q = 0; il + q < jl; ++q) dst[q] = T[jl * PITCH + il + q];
    }
  }
}

template <typename K>
hipError_t launch(K kernel, const GemmArgs& a, hipStream_t stream, int threads = 256) {
  const int64_t grid = (int64_t)a.nprob * a.N * a.tiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <typename K>
hipError_t launch_interleaved(K kernel, const GemmArgs& a, hipStream_t stream, int threads = 256) {
  const int64_t grid = (a.N + 7) / 8 * 8 * a.nprob * a.tiles;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// A stopped block of an adaptive solve (binary16 operands): the accumulators take the operand that
// passes through (X for pass 1, Y for pass 2) at the tile's positions, mapped exactly as the product
// would have staged it (operand_map's arithmetic, element by element).
template <typename TE, int MTM, int MTN, int WTM, int WTN>
__device__ __forceinline__ void pass_tile_f16(const Product& P, const TE* X, const TE* Y, int B, int i0,
                                              int j0, int wm, int wn, int lane, f32x16 (&acc)[MTM][MTN]) {
  const TE* Z = P.pass == 1 ? X : Y;
  const bool map = P.pass == 1 ? P.map_x : P.map_y;
  const TE ma = (TE)P.map_a, mg = (TE)P.map_g;
  const int li = lane & 31, h = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MTM; ++mt)
#pragma unroll
    for (int nt = 0; nt < MTN; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + wm * WTM + mt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = j0 + wn * WTN + nt * 32 + li;
        TE z = Z[(int64_t)i * B + j];
        if (map) {
          z = z * ma;
          if (i == j) z = z + mg;
        }
        acc[mt][nt][r] = (float)z;
      }
}

// kernel launchers of the two precisions
hipError_t launch_f32(GemmArgs& a, Trans trans, bool sym, hipStream_t stream);
hipError_t launch_f16(GemmArgs& a, dash_prec in_prec, dash_prec out_prec, bool sym, bool y_sym, hipStream_t stream);
// fp32 products from three-piece bfloat16 splits (gemm_split.hip), B % 256 == 0: symmetric results
// (sym) of NN with an exactly symmetric right operand, of NT or of TN; general results of NN
hipError_t launch_split(GemmArgs& a, bool sym, Trans trans, bool y_sym, bool h2, hipStream_t stream);

}  // namespace gemm
}  // namespace dash
