// api.hip -- the C ABI of include/dash.h: host-side validation, workspace carving and the solver
// drivers that enqueue the kernels of gemm.hip, scale.hip and elementwise.hip on the caller's stream.
//
// Nothing here allocates device memory or synchronises: every intermediate lives in the caller's
// workspace, and per-block scalars derived from s stay on the device (coefficient table).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <utility>
#include <vector>

#include "dash_internal.hpp"

using namespace dash;

namespace {

#define TRY(x)                                              \
  do {                                                      \
    if ((x) != hipSuccess) return DASH_ERR_DEVICE;          \
  } while (0)

constexpr int64_t MAX_N = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool valid_B(int32_t B) { return B >= 64 && B <= 8192 && B % 64 == 0; }
bool valid_N(int64_t N) { return N >= 1 && N <= MAX_N; }
hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// fp32 storage: DASH_FP32, and DASH_FP32_SPLIT whose operands are split only inside the products
bool fp32_prec(dash_prec p) { return p == DASH_FP32 || p == DASH_FP32_SPLIT; }
size_t elem_size(dash_prec p) { return fp32_prec(p) ? 4 : 2; }
// 2-byte operand formats of the half-precision solvers
bool half_prec(dash_prec p) { return p == DASH_FP16 || p == DASH_BF16; }
size_t stack_bytes(int64_t N, int B, dash_prec p) { return align_up((size_t)N * B * B * elem_size(p), 256); }
size_t coef_bytes(int64_t N) { return align_up((size_t)N * COEF_STRIDE * sizeof(float), 256); }

// Bump allocator over the caller's workspace.
struct Carver {
  char* p;
  size_t left;
  void* take(size_t n) {
    n = align_up(n, 256);
    if (n > left) return nullptr;
    void* r = p;
    p += n;
    left -= n;
    return r;
  }
};

// Stack-sized buffers of the caller's workspace handed out to a solver's iterates.
struct Pool {
  std::vector<void*> free_list;
  void* get() {
    void* r = free_list.back();
    free_list.pop_back();
    return r;
  }
  void put(void* p) { free_list.push_back(p); }
};

size_t flag_bytes(int64_t N) { return align_up((size_t)N * sizeof(int32_t), 256); }
// NDB with two-piece binary16 products: the input's bound per block, and per-wave maxima of every
// tile (8 per 256-wide tile of the block) for each of the five iterate stacks
int64_t ndb_parts(int B) { return (int64_t)(B / 256) * (B / 256) * 8; }
// statistics with two-piece binary16 products: G's bound per tile
size_t ws_stats16(int64_t N) { return align_up((size_t)N * sizeof(float), 256); }
// the statistics' arguments short of prec and workspace
dash_status stats_args_check(const float* G_stack, int64_t NG, int32_t B, float beta, const float* A) {
  if (!G_stack || !A || !aligned(G_stack, 16) || !aligned(A, 16)) return DASH_ERR_INVALID_ARG;
  if (!valid_N(NG) || !valid_N(2 * NG)) return DASH_ERR_INVALID_ARG;
  if (!(beta >= 0.f && beta <= 1.f)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  return DASH_OK;
}
// apply: the intermediate stack T = XL G, and for two-piece binary16 products the bounds of XL, G
// and XR per block and T's per-wave maxima
size_t ws_apply(int64_t N, int B) {
  return stack_bytes(N, B, DASH_FP32) + 3 * align_up((size_t)N * sizeof(float), 256) +
         align_up((size_t)N * ndb_parts(B) * sizeof(float), 256);
}
size_t ndb_bound_bytes(int64_t N, int B) {
  return align_up((size_t)N * sizeof(float), 256) + 5 * align_up((size_t)N * ndb_parts(B) * sizeof(float), 256);
}
size_t ws_ndb(int64_t N, int B) {
  return coef_bytes(N) + flag_bytes(N) + 5 * stack_bytes(N, B, DASH_FP32) + ndb_bound_bytes(N, B);
}
// binary16 NDB: six binary16 stacks for the iterates, reused as three fp32 stacks by the correction,
// and per-block flags and residuals of the guarded correction (at most 16 steps)
size_t ndb_half_region(int64_t N, int B) {
  const size_t h6 = 6 * stack_bytes(N, B, DASH_FP16), f3 = 3 * stack_bytes(N, B, DASH_FP32);
  return h6 > f3 ? h6 : f3;
}
size_t ws_ndb_half(int64_t N, int B) {
  return coef_bytes(N) + 2 * flag_bytes(N) + align_up((size_t)N * 17 * sizeof(float), 256) + ndb_half_region(N, B);
}
size_t ws_cn(int64_t N, int B, dash_prec p) { return coef_bytes(N) + flag_bytes(N) + 5 * stack_bytes(N, B, p); }
size_t cheb_tab_bytes(int64_t N);
// magnitude bounds of the two-piece binary16 Clenshaw products: max |A| per block, and two
// alternating sets of per-wave maxima of b_k (8 waves for each of the block's upper-triangle
// 256-wide tiles)
int64_t amax_parts(int B) {
  const int64_t t = B / 256;
  return t * (t + 1) / 2 * 8;
}
size_t amax_bytes(int64_t N, int B) {
  return align_up((size_t)N * sizeof(float), 256) + 2 * align_up((size_t)N * amax_parts(B) * sizeof(float), 256);
}
size_t ws_cheb(int64_t N, int B) {
  return coef_bytes(N) + cheb_tab_bytes(N) + 2 * stack_bytes(N, B, DASH_FP32) + amax_bytes(N, B);
}
size_t ws_evd(int64_t N, int B) { return evd_workspace_bytes(N, B); }
size_t ws_scale(int64_t N, int B, dash_prec p, int k) { return k == 0 ? 0 : power_workspace_bytes(N, B, p); }
// routed solve: per-block arrays (estimate, probe result, route, freeze, the second solver's status
// and monitor), then one region that the estimate, the Chebyshev solve, the probes and the coupled
// Newton fallback use in turn
constexpr int ROUTED_MAX_CN_ITERS = 64;
size_t ws_routed_arrays(int64_t N) {
  return 2 * align_up((size_t)N * sizeof(float), 256) + 3 * flag_bytes(N) +
         align_up((size_t)N * ROUTED_MAX_CN_ITERS * sizeof(float), 256);
}
size_t ws_routed(int64_t N, int B) {
  size_t region = ws_cheb(N, B);
  const size_t cn = ws_cn(N, B, DASH_FP32), pw = power_workspace_bytes(N, B, DASH_FP32);
  if (cn > region) region = cn;
  if (pw > region) region = pw;
  return ws_routed_arrays(N) + region;
}

Product prod(const void* X, const void* Y, void* D, const float* C = nullptr, const float* E = nullptr,
             void* D2 = nullptr) {
  Product p;
  p.X = X;
  p.Y = Y;
  p.D = D;
  p.C = C;
  p.E = E;
  p.D2 = D2;
  return p;
}

// ------------------------------------------------------------------------------------------------
// Newton-Denman-Beavers: one call on M (optionally M = A / s via the coefficient table).
// Returns the buffer holding the wanted iterate (Y when !want_z) or writes Z into `final_out`
// scaled by coef[final_idx] (when want_z).
// ------------------------------------------------------------------------------------------------
struct NdbCtx {
  int64_t N;
  int B;
  const float* coef;
  float* monitor;  // base of [N, mon_cols] or null
  int mon_cols;
  int32_t* status;
  hipStream_t st;
  Pool* pool;
  // adaptive stopping (null: every block runs all T steps): a block whose monitor is <= tol before
  // step k >= 1 keeps its iterates from then on; steps (optional, stride 2) receives the steps run
  int32_t* freeze = nullptr;
  float tol = 0.f;
  int32_t* steps = nullptr;
  // products formed from three-piece bfloat16 splits (DASH_FP32_SPLIT) where the shape allows
  bool split = false;
  // or from two-piece binary16 splits (DASH_FP32_SPLIT16, B % 256 == 0): every stack an operand
  // comes from has its magnitude bound here (the input's from a pass over it, the products' from
  // the per-wave maxima their launches store, the elementwise results' from a pass)
  struct Bound {
    const void* buf;
    float* amax;
    int parts;
  };
  std::vector<Bound>* bounds = nullptr;
  // the coefficient that unscales the wanted Z into the output: s^{-1/4} for the composed inverse
  // fourth root, s^{-1/2} for one call's inverse square root
  int8_t final_ia = CO_U;
};

dash_status ndb_call(const NdbCtx& c, const float* M, bool m_from_pool, bool scaled, int T, int mon_col,
                     bool want_z, float* final_out, float** y_out) {
  // step 0: Z_0 = I so P_0 = M and S_0 = (3I - M)/2; Y_1 = M S_0 = 1.5 M - 0.5 M^2, Z_1 = S_0.
  const bool last = (T == 1);
  // every product is a general one (NDB iterates are never symmetrised)
  const bool h2 = c.bounds && !c.freeze && c.B % 256 == 0;
  const dash_prec PP = h2 ? DASH_FP32_SPLIT16 : (c.split && !c.freeze && c.B % 256 == 0) ? DASH_FP32_SPLIT : DASH_FP32;
  auto bound = [&](const void* buf) -> NdbCtx::Bound* {
    for (auto& x : *c.bounds)
      if (x.buf == buf) return &x;
    return nullptr;
  };
  // a product's operand bounds, and (when it writes a stack that has them) its per-wave maxima
  auto tag = [&](Product& p) -> bool {
    if (!h2) return true;
    const NdbCtx::Bound* bx = bound(p.X);
    const NdbCtx::Bound* by = bound(p.Y);
    if (!bx || !by || bx->parts < 1 || by->parts < 1) return false;
    p.amax_x = bx->amax;
    p.amax_x_parts = bx->parts;
    p.amax_y = by->amax;
    p.amax_y_parts = by->parts;
    if (NdbCtx::Bound* bd = bound(p.D)) {
      p.amax_d = bd->amax;
      bd->parts = (int)ndb_parts(c.B);
    }
    return true;
  };
  // a stack written by an elementwise kernel: its bound from a pass over it
  auto pass_bound = [&](const void* buf) -> hipError_t {
    if (!h2) return hipSuccess;
    NdbCtx::Bound* bd = bound(buf);
    if (!bd) return hipErrorInvalidValue;
    bd->parts = 1;
    return launch_block_amax((const float*)buf, c.N, c.B, bd->amax, c.st);
  };
  if (c.freeze) TRY(launch_freeze_reset(c.freeze, c.steps, 2, T, c.N, c.st));
  float* Z = nullptr;
  float* Y = nullptr;
  {
    Affine s0;
    s0.X = M;
    s0.a = -0.5f;
    s0.ia = scaled ? CO_R1 : CO_NONE;
    s0.g = 1.5f;
    s0.coef = c.coef;
    if (c.monitor) {  // ||P_0 - I||^2 = 4 ||S_0 - I||^2
      s0.monitor = c.monitor + mon_col;
      s0.mon_stride = c.mon_cols;
      s0.mon_mul = 4.f;
    }
    if (!last || want_z) {
      Z = (float*)c.pool->get();
      s0.D = Z;
      TRY(launch_affine(s0, c.N, c.B, c.st));
      if (!last) TRY(pass_bound(Z));
    } else if (c.monitor) {  // only the monitor is wanted from S_0: write it to a scratch buffer
      float* tmp = (float*)c.pool->get();
      s0.D = tmp;
      TRY(launch_affine(s0, c.N, c.B, c.st));
      c.pool->put(tmp);
    }
  }
  if (!last || !want_z) {
    Y = (float*)c.pool->get();
    Epilogue e;
    e.alpha = -0.5f;
    e.ia = scaled ? CO_R2 : CO_NONE;
    e.beta = 1.5f;
    e.ib = scaled ? CO_R1 : CO_NONE;
    e.coef = c.coef;
    Product p = prod(M, M, Y, M);
    if (!tag(p)) return DASH_ERR_INVALID_ARG;
    TRY(launch_gemm(&p, 1, c.N, c.B, PP, DASH_FP32, Trans::NN, false, e, c.st));
  }
  if (m_from_pool) c.pool->put((void*)M);
  if (last) {
    if (want_z) {
      Affine fin;  // X = u Z_1
      fin.X = Z;
      fin.D = final_out;
      fin.a = 1.f;
      fin.ia = c.final_ia;
      fin.coef = c.coef;
      fin.status = c.status;
      TRY(launch_affine(fin, c.N, c.B, c.st));
      c.pool->put(Z);
    } else {
      *y_out = Y;
    }
    return DASH_OK;
  }
  for (int k = 1; k < T; ++k) {
    // S = (3I - Z Y) / 2, monitor ||Z Y - I|| = 2 ||S - I||
    float* S = (float*)c.pool->get();
    {
      Epilogue e;
      e.alpha = -0.5f;
      e.gamma = 1.5f;
      if (c.monitor) {
        e.monitor = c.monitor + mon_col + k;
        e.mon_stride = c.mon_cols;
        e.mon_mul = 4.f;
      }
      Product p = prod(Z, Y, S);
      p.freeze = c.freeze;  // a stopped block needs no S
      if (!tag(p)) return DASH_ERR_INVALID_ARG;
      TRY(launch_gemm(&p, 1, c.N, c.B, PP, DASH_FP32, Trans::NN, false, e, c.st));
    }
    if (c.freeze)
      TRY(launch_freeze_update(c.monitor, c.mon_cols, mon_col + k, c.B, c.tol, c.freeze, c.steps, 2, k, c.N, c.st));
    if (k == T - 1) {
      if (want_z) {  // Z_T = S Z, unscaled into the output
        Epilogue e;
        e.alpha = 1.f;
        e.ia = c.final_ia;
        e.coef = c.coef;
        e.status = c.status;
        Product p = prod(S, Z, final_out);
        p.freeze = c.freeze;
        p.pass = 2;
        if (!tag(p)) return DASH_ERR_INVALID_ARG;
        TRY(launch_gemm(&p, 1, c.N, c.B, PP, DASH_FP32, Trans::NN, false, e, c.st));
        c.pool->put(Y);
        c.pool->put(Z);
      } else {  // Y_T = Y S
        float* Yn = (float*)c.pool->get();
        Epilogue e;
        Product p = prod(Y, S, Yn);
        p.freeze = c.freeze;
        p.pass = 1;
        if (!tag(p)) return DASH_ERR_INVALID_ARG;
        TRY(launch_gemm(&p, 1, c.N, c.B, PP, DASH_FP32, Trans::NN, false, e, c.st));
        c.pool->put(Y);
        c.pool->put(Z);
        *y_out = Yn;
      }
      c.pool->put(S);
      return DASH_OK;
    }
    float* Yn = (float*)c.pool->get();
    float* Zn = (float*)c.pool->get();
    Epilogue e;
    Product p[2] = {prod(Y, S, Yn), prod(S, Z, Zn)};
    p[0].freeze = p[1].freeze = c.freeze;
    p[0].pass = 1;
    p[1].pass = 2;
    if (!tag(p[0]) || !tag(p[1])) return DASH_ERR_INVALID_ARG;
    TRY(launch_gemm(p, 2, c.N, c.B, PP, DASH_FP32, Trans::NN, false, e, c.st));
    c.pool->put(Y);
    c.pool->put(Z);
    c.pool->put(S);
    Y = Yn;
    Z = Zn;
  }
  return DASH_OK;
}

// One NDB call with 2-byte iterates H (binary16 or bfloat16; fp32 accumulation) on the stack M in
// that format: every stored iterate is rounded to H once, by the epilogue that forms it.  Step 0: S_0 = (3I - M)/2 is
// Z_1 and Y_1 = M S_0.  Returns Y_T (binary16) in *y_out, or (want_z) writes Z_T in fp32 into
// final_out, scaled by coef[final_ia], with the finite check into status.  Monitor as in ndb_call.
dash_status ndb_half_call(const NdbCtx& c, dash_prec H, void* M, bool m_from_pool, int T, int mon_col, bool want_z,
                          float* final_out, int8_t final_ia, void** y_out) {
  void* Z = c.pool->get();
  {
    Affine s0;
    s0.X = M;
    s0.x_prec = H;
    s0.D = Z;
    s0.d_prec = H;
    s0.a = -0.5f;
    s0.g = 1.5f;
    if (c.monitor) {  // ||P_0 - I||^2 = 4 ||S_0 - I||^2
      s0.monitor = c.monitor + mon_col;
      s0.mon_stride = c.mon_cols;
      s0.mon_mul = 4.f;
    }
    TRY(launch_affine(s0, c.N, c.B, c.st));
  }
  if (T == 1 && want_z) {  // Z_1 = S_0
    Affine fin;
    fin.X = Z;
    fin.x_prec = H;
    fin.D = final_out;
    fin.a = 1.f;
    fin.ia = final_ia;
    fin.coef = c.coef;
    fin.status = c.status;
    TRY(launch_affine(fin, c.N, c.B, c.st));
    c.pool->put(Z);
    if (m_from_pool) c.pool->put(M);
    return DASH_OK;
  }
  void* Y = c.pool->get();
  {
    Product p = prod(M, Z, Y);
    TRY(launch_gemm(&p, 1, c.N, c.B, H, H, Trans::NN, false, Epilogue(), c.st));
  }
  if (m_from_pool) c.pool->put(M);
  if (T == 1) {
    c.pool->put(Z);
    *y_out = Y;
    return DASH_OK;
  }
  for (int k = 1; k < T; ++k) {
    void* S = c.pool->get();
    {
      Epilogue e;  // S = (3I - Z Y) / 2, monitor ||Z Y - I|| = 2 ||S - I||
      e.alpha = -0.5f;
      e.gamma = 1.5f;
      if (c.monitor) {
        e.monitor = c.monitor + mon_col + k;
        e.mon_stride = c.mon_cols;
        e.mon_mul = 4.f;
      }
      Product p = prod(Z, Y, S);
      TRY(launch_gemm(&p, 1, c.N, c.B, H, H, Trans::NN, false, e, c.st));
    }
    if (k == T - 1) {
      if (want_z) {
        Epilogue e;
        e.ia = final_ia;
        e.coef = c.coef;
        e.status = c.status;
        Product p = prod(S, Z, final_out);
        TRY(launch_gemm(&p, 1, c.N, c.B, H, DASH_FP32, Trans::NN, false, e, c.st));
        c.pool->put(Y);
      } else {
        void* Yn = c.pool->get();
        Product p = prod(Y, S, Yn);
        TRY(launch_gemm(&p, 1, c.N, c.B, H, H, Trans::NN, false, Epilogue(), c.st));
        c.pool->put(Y);
        *y_out = Yn;
      }
      c.pool->put(Z);
      c.pool->put(S);
      return DASH_OK;
    }
    void* Yn = c.pool->get();
    void* Zn = c.pool->get();
    Product p[2] = {prod(Y, S, Yn), prod(S, Z, Zn)};
    TRY(launch_gemm(p, 2, c.N, c.B, H, H, Trans::NN, false, Epilogue(), c.st));
    c.pool->put(Y);
    c.pool->put(Z);
    c.pool->put(S);
    Y = Yn;
    Z = Zn;
  }
  return DASH_OK;
}

// Interval of the Chebyshev solve per block, in units of A_b / s_b: [lo_rel, hi] for every block
// when lo_rel > 0, else [max(floor, theta lam[b]) / s_b, hi].
struct ChebInterval {
  double lo_rel = 0.0, floor = 0.0, hi = 1.0;
  const float* lam = nullptr;
  float theta = 1.f;
};

size_t cheb_tab_bytes(int64_t N) {
  return align_up((size_t)N * COEF_STRIDE * sizeof(float) * (CHEB_MAX_DEGREE - 1), 256);
}

// The Clenshaw recurrence on A/s with the per-block plan of launch_cheb_plan: b_{d+1} = b_{d+2} = 0,
// b_k = c_k I + 2 T b_{k+1} - b_{k+2} (k = d .. 1), X = s^{-1/4} (c_0 I + T b_1 - b_2),
// T = (2 A/s - (hi + lo) I) / (hi - lo); d - 1 products, each epilogue reading its launch's row of
// the plan.  b_d and b_{d-1} are never stored: the first product reads A mapped to b_{d-1} (or, with
// split products, is written as a product of A with itself), and the second takes A as b_{k+2}.
dash_status cheb_impl(const float* A, const float* s, int64_t N, int32_t B, int32_t degree, const ChebInterval& iv,
                      dash_prec prec, float* X, float* lo_out, int32_t* status, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!fp32_prec(prec) && prec != DASH_FP32_SPLIT16) return DASH_ERR_INVALID_ARG;
  if (!A || !s || !X || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (X == A || degree < 1 || degree > CHEB_MAX_DEGREE) return DASH_ERR_INVALID_ARG;
  if ((status && !aligned(status, 4)) || (lo_out && !aligned(lo_out, 4))) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_cheb(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* coef = (float*)cv.take(coef_bytes(N));
  float* tab = (float*)cv.take(cheb_tab_bytes(N));
  float* b1 = (float*)cv.take(stack_bytes(N, B, DASH_FP32));
  float* b2 = (float*)cv.take(stack_bytes(N, B, DASH_FP32));
  float* amax_a = (float*)cv.take(align_up((size_t)N * sizeof(float), 256));
  float* amax_slot[2];
  for (int i = 0; i < 2; ++i) amax_slot[i] = (float*)cv.take(align_up((size_t)N * amax_parts(B) * sizeof(float), 256));
  const int d = degree;
  // split products need 256-wide tiles and an exactly symmetric right operand: every b_{k+1} is
  // stored mirrored; the first product maps A on the fp32 cores unless it can be written as
  // (alpha a1/s)(A + c I) A (degree >= 3), which the split kernel forms with A read by columns
  const bool split = (prec == DASH_FP32_SPLIT || prec == DASH_FP32_SPLIT16) && B % 256 == 0;
  const bool split_first = split && d >= 3;
  // two-piece binary16 products (from the first product on, degree >= 3): launch q scales its left
  // operand A + c I by max |A| + |c| and its right one by max |A| (q = 0) or by the largest of the
  // per-wave maxima that launch q - 1 stored in set (q - 1) % 2; its own go to set q % 2
  const bool h2 = split_first && prec == DASH_FP32_SPLIT16;
  const dash_prec sp_prec = h2 ? DASH_FP32_SPLIT16 : DASH_FP32_SPLIT;
  auto bounds = [&](Product& pr, int q, bool last) {
    if (!h2) return;
    pr.amax_x = amax_a;
    pr.amax_y = q == 0 ? amax_a : amax_slot[(q - 1) % 2];
    pr.amax_y_parts = q == 0 ? 1 : (int)amax_parts(B);
    pr.amax_d = last ? nullptr : amax_slot[q % 2];
  };
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  TRY(launch_coef(s, N, coef, status, st));
  {
    ChebPlan cp;
    cp.N = N;
    cp.d = d;
    cp.split_first = split_first;
    cp.s = s;
    cp.coef = coef;
    cp.lo_rel = iv.lo_rel;
    cp.floor = iv.floor;
    cp.lam = iv.lam;
    cp.theta = iv.theta;
    cp.hi = iv.hi;
    cp.tab = tab;
    cp.lo_out = lo_out;
    cp.status = status;
    TRY(launch_cheb_plan(cp, st));
  }
  auto row = [&](int q) { return (const float*)(tab + (int64_t)q * N * COEF_STRIDE); };
  if (d == 1) {
    Affine fin;
    fin.X = A;
    fin.D = X;
    fin.a = 1.f;
    fin.ia = CS_ALPHA;
    fin.g = 1.f;
    fin.ig = CS_GAMMA;
    fin.coef = row(0);
    fin.status = status;
    TRY(launch_affine(fin, N, B, st));
    return DASH_OK;
  }
  // launch q's epilogue: every coefficient from its row of the plan (C = b_{k+1} folded)
  auto epi = [&](int q, bool last) {
    Epilogue e;
    e.coef = row(q);
    e.alpha = 1.f;
    e.ia = CS_ALPHA;
    e.beta = 1.f;
    e.ib = CS_BETA;
    e.gamma = 1.f;
    e.ig = CS_GAMMA;
    e.delta = 1.f;
    e.id = CS_DELTA;
    e.fold_c = true;
    e.c_over_a = 1.f;
    e.ic = CS_COVERA;
    if (last) e.status = status;
    return e;
  };
  auto run = [&](Product& pr, const Epilogue& e) {
    const bool sp = split && !pr.map_y;
    return launch_gemm(&pr, 1, N, B, sp ? sp_prec : DASH_FP32, DASH_FP32, Trans::NN, true, e, st, sp);
  };
  if (h2) TRY(launch_block_amax(A, N, B, amax_a, st));
  // the first product: k = d - 2 (or the final one when d == 2); b_{k+2} = b_d = c_d I rides in gamma
  if (split_first) {
    Product pr = prod(A, A, b2, A);
    bounds(pr, 0, false);
    Epilogue e = epi(0, false);
    TRY(launch_gemm(&pr, 1, N, B, sp_prec, DASH_FP32, Trans::NN, true, e, st, false));
  } else {
    const bool last = (d == 2);
    Product pr = prod(A, A, last ? (void*)X : (void*)b2, A, nullptr);
    pr.map_y = true;
    pr.map_a = 1.f;
    pr.map_ia = CS_MAPA;
    pr.map_g = 1.f;
    pr.map_ig = CS_MAPG;
    TRY(run(pr, epi(0, last)));
    if (last) return DASH_OK;
  }
  // the second product: k = d - 3 (or the final one when d == 3), b_{k+2} = b_{d-1} read as A
  // (A is symmetric, so its upper-triangle tiles serve)
  {
    const bool last = (d == 3);
    Product pr = prod(A, b2, last ? (void*)X : (void*)b1, b2, A);
    bounds(pr, 1, last);
    TRY(run(pr, epi(1, last)));
    if (last) return DASH_OK;
  }
  // b_{d-3} is in b1 and b_{d-2} in b2, i.e. b1 = b_{k+1} and b2 = b_{k+2} for k = d - 4; from here
  // on b_k is written over b_{k+2}
  int q = 2;
  for (int k = d - 4; k >= 1; --k, ++q) {
    Product pr = prod(A, b1, b2, b1, b2);
    bounds(pr, q, false);
    TRY(run(pr, epi(q, false)));
    std::swap(b1, b2);
  }
  Product pr = prod(A, b1, X, b1, b2);
  bounds(pr, q, true);
  TRY(run(pr, epi(q, true)));
  return DASH_OK;
}

dash_status check_mats(const dash_mat* m, int32_t n, int32_t B, int64_t* tiles) {
  if (!m || n < 1) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  int64_t t = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (!m[i].ptr || !aligned(m[i].ptr, 16) || m[i].ld % 4 != 0) return DASH_ERR_INVALID_ARG;
    if (m[i].rows < 1 || m[i].cols < 1 || m[i].ld < m[i].cols) return DASH_ERR_INVALID_ARG;
    t += ((m[i].rows + B - 1) / B) * ((m[i].cols + B - 1) / B);
  }
  *tiles = t;
  return DASH_OK;
}


// Coupled Newton with 2-byte iterates H (binary16 or bfloat16; T >= 2), on M_0 = A/s already stored
// in M0 in that format.
// S_k = (5I - M_k)/4 is never stored: every product that takes S_k reads M_k and maps it as it is
// staged (operand map -1/4 Z + 5/4 I, the same single rounding a binary16 elementwise pass would
// apply), and X_1 = S_0 is likewise M_0 mapped.  M_0 stays alive until X_2 has been formed.
// freeze (optional, adaptive): a block whose monitor ||M_k - I|| is <= tol before step k >= 1 keeps
// X_k from then on (its later products are skipped or pass X through).
dash_status cn_half(dash_prec H, int64_t N, int B, int T, float* X, float* monitor, int32_t* status, const float* coef,
                    void* M0, Pool& pool, hipStream_t st, int32_t* freeze, float tol, int32_t* steps) {
  auto mapped = [](Product p, bool mx, bool my) {
    p.map_x = mx;
    p.map_y = my;
    p.map_a = -0.25f;
    p.map_g = 1.25f;
    return p;
  };
  auto frozen = [&](Product p, int8_t pass) {
    p.freeze = freeze;
    p.pass = pass;
    return p;
  };
  void* M = M0;
  void* Xk = nullptr;  // null while X_k = S_0 (k = 1) is M_0 mapped
  for (int k = 0; k < T; ++k) {
    if (freeze && k >= 1)  // monitor column k (||M_k - I||) is complete
      TRY(launch_freeze_update(monitor, T, k, B, tol, freeze, steps, 1, k, N, st));
    if (k == T - 1) {  // X_T = s^{-1/4} X_{T-1} S_{T-1}, fp32 output
      Epilogue e;
      e.ia = CO_U;
      e.coef = coef;
      e.status = status;
      Product pr = frozen(mapped(prod(Xk ? Xk : M0, M, X), Xk == nullptr, true), 1);
      TRY(launch_gemm(&pr, 1, N, B, H, DASH_FP32, Trans::NN, true, e, st, true));
      break;
    }
    void* S2 = pool.get();
    if (k == 0) {
      Product pr = mapped(prod(M, M, S2), true, true);
      TRY(launch_gemm(&pr, 1, N, B, H, H, Trans::NN, true, Epilogue(), st, true));
    } else {  // X_{k+1} = X_k S_k and S_k^2 in one launch
      void* Xn = pool.get();
      Product pr[2] = {frozen(mapped(prod(Xk ? Xk : M0, M, Xn), Xk == nullptr, true), 1),
                       frozen(mapped(prod(M, M, S2), true, true), 0)};
      TRY(launch_gemm(pr, 2, N, B, H, H, Trans::NN, true, Epilogue(), st, true));
      pool.put(Xk ? Xk : M0);  // X_k (or M_0, whose last use as X_1 this was) is dead
      Xk = Xn;
    }
    void* S4 = pool.get();
    {
      Product pr = frozen(prod(S2, S2, S4), 0);
      TRY(launch_gemm(&pr, 1, N, B, H, H, Trans::NN, true, Epilogue(), st, true));
    }
    pool.put(S2);
    Epilogue e;
    if (monitor) {
      e.monitor = monitor + (k + 1);
      e.mon_stride = T;
    }
    void* Mn = pool.get();
    Product pr = frozen(prod(M, S4, Mn), 0);
    TRY(launch_gemm(&pr, 1, N, B, H, H, Trans::NN, true, e, st, true));
    if (M != M0) pool.put(M);  // M_0 is released with X_1 above
    pool.put(S4);
    M = Mn;
  }
  if (monitor) TRY(launch_monitor_finish(monitor, N * T, B, st));
  return DASH_OK;
}

}  // namespace

extern "C" {

int32_t dash_abi_version(void) { return DASH_ABI_VERSION; }

const char* dash_status_string(dash_status s) {
  switch (s) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARG: return "invalid argument";
    case DASH_ERR_SHAPE: return "unsupported shape";
    case DASH_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DASH_ERR_UNSUPPORTED: return "unsupported request";
    case DASH_ERR_DEVICE: return "HIP launch failed";
  }
  return "unknown status";
}

int64_t dash_solver_products(dash_op op, int32_t iters1, int32_t iters2) {
  switch (op) {
    case DASH_OP_NDB:
      if (iters1 < 1 || iters2 < 1) return -1;
      return (iters1 == 1 ? 1 : 3 * (int64_t)iters1 - 3) + (3 * (int64_t)iters2 - 3);
    case DASH_OP_CN:
      if (iters1 < 1) return -1;
      return iters1 == 1 ? 0 : 4 * (int64_t)iters1 - 4;
    case DASH_OP_CHEB:
      if (iters1 < 1) return -1;
      return iters1 < 2 ? 0 : (int64_t)iters1 - 1;
    default: return -1;
  }
}

double dash_flops(dash_op op, int64_t N, int32_t B, dash_prec prec, int32_t a1, int32_t a2) {
  if (prec == DASH_FP32_SPLIT16) prec = DASH_FP32_SPLIT;  // the same tiles
  if (!valid_N(N) || !valid_B(B) || (!fp32_prec(prec) && !half_prec(prec))) return -1.0;
  const bool split = prec == DASH_FP32_SPLIT && B % 256 == 0;
  if (prec == DASH_FP32_SPLIT) prec = DASH_FP32;
  const double full = 2.0 * B * B * (double)B * (double)N;
  // fraction of the tiles a triangle-only product computes, for the tile width the kernels use
  auto tri = [&](dash_prec p) {
    const int tile = (half_prec(p) && B % 256 == 0) ? 256 : (B % 128 == 0 ? 128 : 64);
    const double t = B / tile;
    return (t * (t + 1) / 2) / (t * t);
  };
  int64_t n;
  switch (op) {
    case DASH_OP_NDB:
      n = dash_solver_products(op, a1, a2);
      return n < 0 ? -1.0 : n * full;
    case DASH_OP_CN:
      n = dash_solver_products(op, a1, 0);
      return n < 0 ? -1.0 : n * full * (half_prec(prec) ? tri(prec) : 1.0);
    case DASH_OP_CHEB:
      n = dash_solver_products(op, a1, 0);
      if (n < 0) return -1.0;
      if (split && n > 1) {  // every product on 256-wide tiles (degree >= 3)
        const double t = B / 256;
        return full * n * (t * (t + 1) / 2) / (t * t);
      }
      return n * full * tri(DASH_FP32);
    case DASH_OP_APPLY: return 2.0 * full;
    case DASH_OP_STATS: return 2.0 * full * tri(DASH_FP32);
    case DASH_OP_SCALE: return a1 < 1 ? -1.0 : 2.0 * B * (double)B * 32.0 * a1 * (double)N;
    case DASH_OP_ROUTED: return -1.0;  // the work depends on the routing the data decides
    case DASH_OP_EVD: {
      // per round: P(P-1)/2 off-pair blocks (two 64^3 products) and P * B/64 eigenvector tiles (one);
      // B/32 - 1 rounds per sweep; then X = Y Y^T (triangle-only)
      if (a1 < 1) return -1.0;
      const double P = B / 64, prod64 = 2.0 * 64 * 64 * 64;
      const double round = (P * (P - 1) / 2 * 2 + P * (B / 64)) * prod64;
      return a1 * (B / 32 - 1) * round * (double)N + full * tri(DASH_FP32);
    }
  }
  return -1.0;
}

dash_status dash_workspace_size(dash_op op, int64_t N, int32_t B, dash_prec prec, int32_t k_or_degree,
                                size_t* bytes) {
  if (!bytes || !valid_N(N)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!fp32_prec(prec) && !half_prec(prec) && prec != DASH_FP32_SPLIT16) return DASH_ERR_INVALID_ARG;
  const bool split16 = prec == DASH_FP32_SPLIT16;
  if (prec == DASH_FP32_SPLIT || prec == DASH_FP32_SPLIT16) prec = DASH_FP32;
  switch (op) {
    case DASH_OP_SCALE:
      if (prec == DASH_BF16) return DASH_ERR_UNSUPPORTED;
      if (k_or_degree < 0 || k_or_degree > 32) return DASH_ERR_INVALID_ARG;
      *bytes = ws_scale(N, B, prec, k_or_degree);
      return DASH_OK;
    case DASH_OP_NDB: *bytes = half_prec(prec) ? ws_ndb_half(N, B) : ws_ndb(N, B); return DASH_OK;
    case DASH_OP_CN: *bytes = ws_cn(N, B, prec); return DASH_OK;
    case DASH_OP_CHEB: *bytes = ws_cheb(N, B); return DASH_OK;
    case DASH_OP_ROUTED: *bytes = ws_routed(N, B); return DASH_OK;
    case DASH_OP_APPLY: *bytes = ws_apply(N, B); return DASH_OK;
    case DASH_OP_STATS: *bytes = split16 ? ws_stats16(N) : 0; return DASH_OK;
    case DASH_OP_EVD: *bytes = ws_evd(N, B); return DASH_OK;
  }
  return DASH_ERR_INVALID_ARG;
}

dash_status dash_stack(const dash_mat* grads, int32_t n, int32_t B, float* G_stack, void* stream) {
  int64_t tiles = 0;
  dash_status st = check_mats(grads, n, B, &tiles);
  if (st != DASH_OK) return st;
  if (!G_stack || !aligned(G_stack, 16)) return DASH_ERR_INVALID_ARG;
  TRY(launch_tile_copy(grads, n, B, G_stack, true, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_unstack(const float* U_stack, int32_t B, const dash_mat* outs, int32_t n, void* stream) {
  int64_t tiles = 0;
  dash_status st = check_mats(outs, n, B, &tiles);
  if (st != DASH_OK) return st;
  if (!U_stack || !aligned(U_stack, 16)) return DASH_ERR_INVALID_ARG;
  TRY(launch_tile_copy(outs, n, B, const_cast<float*>(U_stack), false, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_update_stats(const float* G_stack, int64_t NG, int32_t B, float beta, float* A, void* stream) {
  return dash_update_stats_prec(G_stack, NG, B, beta, DASH_FP32, A, stream);
}

dash_status dash_update_stats_prec(const float* G_stack, int64_t NG, int32_t B, float beta, dash_prec prec, float* A,
                                   void* stream) {
  if (!fp32_prec(prec)) return DASH_ERR_INVALID_ARG;
  const dash_status chk = stats_args_check(G_stack, NG, B, beta, A);
  if (chk != DASH_OK) return chk;
  float* L = A;
  float* R = A + NG * (int64_t)B * B;
  Epilogue e;
  e.alpha = 1.f - beta;
  e.beta = beta;
  const dash_prec pp = (prec == DASH_FP32_SPLIT && B % 256 == 0) ? DASH_FP32_SPLIT : DASH_FP32;
  Product pl = prod(G_stack, G_stack, L, L);  // G G^T : Y read transposed
  TRY(launch_gemm(&pl, 1, NG, B, pp, DASH_FP32, Trans::NT, true, e, as_stream(stream)));
  Product pr = prod(G_stack, G_stack, R, R);  // G^T G : X read transposed
  TRY(launch_gemm(&pr, 1, NG, B, pp, DASH_FP32, Trans::TN, true, e, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_update_stats_ws(const float* G_stack, int64_t NG, int32_t B, float beta, dash_prec prec, float* A,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (prec != DASH_FP32_SPLIT16) return dash_update_stats_prec(G_stack, NG, B, beta, prec, A, stream);
  const dash_status chk = stats_args_check(G_stack, NG, B, beta, A);
  if (chk != DASH_OK) return chk;
  if (B % 256 != 0) return dash_update_stats_prec(G_stack, NG, B, beta, DASH_FP32, A, stream);
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_stats16(NG)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  // both products read G on both sides: one bound per tile serves all four operands
  float* bound = (float*)ws;
  TRY(launch_block_amax(G_stack, NG, B, bound, st));
  float* L = A;
  float* R = A + NG * (int64_t)B * B;
  Epilogue e;
  e.alpha = 1.f - beta;
  e.beta = beta;
  Product pl = prod(G_stack, G_stack, L, L);  // G G^T : Y's rows as B's columns
  pl.amax_x = pl.amax_y = bound;
  TRY(launch_gemm(&pl, 1, NG, B, DASH_FP32_SPLIT16, DASH_FP32, Trans::NT, true, e, st));
  Product pr = prod(G_stack, G_stack, R, R);  // G^T G : both operands' columns gathered
  pr.amax_x = pr.amax_y = bound;
  TRY(launch_gemm(&pr, 1, NG, B, DASH_FP32_SPLIT16, DASH_FP32, Trans::TN, true, e, st));
  return DASH_OK;
}

}  // extern "C"

namespace dash {
// Argument checks of dash_scale short of the workspace (shared with dash_scale_noalloc).
dash_status scale_args_check(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                             int32_t steps, const float* V0, const float* s) {
  if (!A || !s || !aligned(A, 16) || !aligned(s, 4) || !valid_N(N)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (how == DASH_SCALE_FROBENIUS) return DASH_OK;
  if (how != DASH_SCALE_POWER) return DASH_ERR_INVALID_ARG;
  if (prec == DASH_BF16) return DASH_ERR_UNSUPPORTED;  // power iteration streams fp32 or binary16 operands
  if (prec != DASH_FP32 && prec != DASH_FP32_SPLIT && prec != DASH_FP16) return DASH_ERR_INVALID_ARG;
  if (k < 1 || k > 32 || steps < 1 || steps > 10000 || !aligned(V0, 4)) return DASH_ERR_INVALID_ARG;
  return DASH_OK;
}
}  // namespace dash

extern "C" {

dash_status dash_start_vectors(int32_t B, int32_t k, uint64_t seed, float* V0, void* stream) {
  if (!V0 || !aligned(V0, 4) || k < 1 || k > 32) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  TRY(launch_start_pool(seed, (int64_t)B * k, V0, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_scale(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                       int32_t steps, const float* V0, uint64_t seed, float* s, void* ws, size_t ws_bytes,
                       void* stream) {
  const dash_status chk = scale_args_check(A, N, B, how, prec, k, steps, V0, s);
  if (chk != DASH_OK) return chk;
  if (how == DASH_SCALE_FROBENIUS) {
    TRY(launch_frobenius(A, N, B, s, as_stream(stream)));
    return DASH_OK;
  }
  if (!ws || !aligned(ws, 256) || ws_bytes < power_workspace_bytes(N, B, prec)) return DASH_ERR_WORKSPACE;
  Carver cv{(char*)ws, ws_bytes};
  PowerPlan p;
  p.N = N;
  p.B = B;
  p.k = k;
  p.steps = steps;
  p.prec = prec;
  p.A = A;
  p.V0 = V0;
  p.seed = seed;
  p.s = s;
  const int RB = B / 64;
  for (int q = 0; q < 2; ++q) p.W[q] = (float*)cv.take((size_t)N * B * 32 * sizeof(float));
  for (int q = 0; q < 2; ++q) p.part[q] = (float*)cv.take((size_t)N * RB * 3 * 32 * sizeof(float));
  p.V0p = (float*)cv.take((size_t)B * 32 * sizeof(float));
  p.coef = (float*)cv.take((size_t)N * COEF_STRIDE * sizeof(float));
  p.Ah = prec == DASH_FP16 ? (_Float16*)cv.take((size_t)N * B * B * sizeof(_Float16)) : nullptr;
  TRY(launch_power_iteration(p, as_stream(stream)));
  return DASH_OK;
}

}  // extern "C"

namespace {

// adaptive stopping of an NDB or CN call: tol < 0 runs every step
struct Stop {
  float tol = -1.f;
  int32_t* steps = nullptr;
  // routed calls: the caller's freeze array, already set (2 = a block this call must leave alone,
  // 0 = a block to solve); no reset and no step counts
  int32_t* freeze_ext = nullptr;
};

dash_status ndb_impl(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1, int32_t iters2, float* X,
                     float* sqrt_out, float* monitor, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                     const Stop& stop, dash_prec prec = DASH_FP32) {
  if (!fp32_prec(prec) && prec != DASH_FP32_SPLIT16) return DASH_ERR_INVALID_ARG;
  if (!A || !s || !X || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (sqrt_out && (!aligned(sqrt_out, 16) || sqrt_out == A || sqrt_out == X)) return DASH_ERR_INVALID_ARG;
  if (X == A || iters1 < 1 || iters2 < 1 || iters1 > 1000 || iters2 > 1000) return DASH_ERR_INVALID_ARG;
  if (monitor && !aligned(monitor, 4)) return DASH_ERR_INVALID_ARG;
  if (status && !aligned(status, 4)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_ndb(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* coef = (float*)cv.take(coef_bytes(N));
  int32_t* freeze = (int32_t*)cv.take(flag_bytes(N));
  Pool pool;
  for (int q = 0; q < 5; ++q) pool.put(cv.take(stack_bytes(N, B, DASH_FP32)));
  // two-piece binary16 products: the bound of A (a pass over it) and of each iterate stack
  std::vector<NdbCtx::Bound> bounds;
  const bool h2 = prec == DASH_FP32_SPLIT16 && B % 256 == 0 && stop.tol < 0.f;
  float* amax_a = (float*)cv.take(align_up((size_t)N * sizeof(float), 256));
  bounds.push_back({A, amax_a, 1});
  for (int q = 0; q < 5; ++q)
    bounds.push_back({pool.free_list[q], (float*)cv.take(align_up((size_t)N * ndb_parts(B) * sizeof(float), 256)), 0});
  const int cols = iters1 + iters2;
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  if (monitor) TRY(launch_fill_f32(monitor, N * cols, 0.f, st));
  TRY(launch_coef(s, N, coef, status, st));
  NdbCtx c{N, B, coef, monitor, cols, status, st, &pool};
  c.split = prec == DASH_FP32_SPLIT;
  if (h2) {
    c.bounds = &bounds;
    TRY(launch_block_amax(A, N, B, amax_a, st));
  }
  if (stop.tol >= 0.f) {
    c.freeze = freeze;
    c.tol = stop.tol;
    c.steps = stop.steps;
  }
  float* Y = nullptr;
  dash_status r = ndb_call(c, A, false, true, iters1, 0, false, nullptr, &Y);
  if (r != DASH_OK) return r;
  if (sqrt_out) {
    Affine sq;
    sq.X = Y;
    sq.D = sqrt_out;
    sq.a = 1.f;
    sq.ia = CO_SQ;
    sq.coef = coef;
    TRY(launch_affine(sq, N, B, st));
  }
  if (c.steps) c.steps += 1;  // the second call's column
  r = ndb_call(c, Y, true, false, iters2, iters1, true, X, nullptr);
  if (r != DASH_OK) return r;
  if (monitor) TRY(launch_monitor_finish(monitor, N * cols, B, st));
  return DASH_OK;
}

// NDB with 2-byte iterates H and the guarded fp32 correction (dash_inverse_root_ndb_half /
// dash_inverse_root_ndb_lowp)
dash_status ndb_lowp_impl(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1, int32_t iters2,
                          dash_prec H, int32_t refine, float* X, float* monitor, int32_t* status, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!A || !s || !X || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (!half_prec(H)) return DASH_ERR_INVALID_ARG;
  if (X == A || iters1 < 1 || iters2 < 1 || iters1 > 1000 || iters2 > 1000 || refine < 0 || refine > 16)
    return DASH_ERR_INVALID_ARG;
  if ((monitor && !aligned(monitor, 4)) || (status && !aligned(status, 4))) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_ndb_half(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* coef = (float*)cv.take(coef_bytes(N));
  int32_t* freeze = (int32_t*)cv.take(flag_bytes(N));
  int32_t* accept = (int32_t*)cv.take(flag_bytes(N));
  float* res = (float*)cv.take((size_t)N * 17 * sizeof(float));  // residual sums of squares per step
  char* region = (char*)cv.take(ndb_half_region(N, B));
  Pool pool;
  for (int q = 1; q < 6; ++q) pool.put(region + q * stack_bytes(N, B, H));
  void* M = region;  // M = h(A / s), the first call's input (not from the pool)
  const int cols = iters1 + iters2;
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  if (monitor) TRY(launch_fill_f32(monitor, N * cols, 0.f, st));
  TRY(launch_coef(s, N, coef, status, st));
  {
    Affine m;
    m.X = A;
    m.D = M;
    m.d_prec = H;
    m.a = 1.f;
    m.ia = CO_R1;
    m.coef = coef;
    TRY(launch_affine(m, N, B, st));
  }
  NdbCtx c{N, B, coef, monitor, cols, status, st, &pool};
  void* Y = nullptr;
  dash_status r = ndb_half_call(c, H, M, false, iters1, 0, false, nullptr, CO_NONE, &Y);
  if (r != DASH_OK) return r;
  // the second call's Z_T in fp32: unscaled into X when there is no correction, else the
  // correction's start
  r = ndb_half_call(c, H, Y, true, iters2, iters1, true, X, refine ? CO_NONE : CO_U, nullptr);
  if (r != DASH_OK) return r;
  if (monitor) TRY(launch_monitor_finish(monitor, N * cols, B, st));
  if (!refine) return DASH_OK;
  // Guarded correction in fp32 against A_s = A / s.  T(X) = (5I - X^4 A_s)/4 carries the residual
  // ||X^4 A_s - I||^2 = 16 ||T(X) - I||^2 in its epilogue.  A step forms the candidate
  // sym(X T(X)), evaluates T of it, and a block takes it only if its residual went down; a block
  // whose residual did not is left at its best X and skips the remaining steps.
  float* R[3] = {(float*)region, (float*)(region + stack_bytes(N, B, DASH_FP32)),
                 (float*)(region + 2 * stack_bytes(N, B, DASH_FP32))};
  TRY(launch_fill_i32(freeze, N, 0, st));
  TRY(launch_fill_f32(res, N * 17, 0.f, st));
  auto evaluate = [&](const float* Xe, float* Tout, float* W0, float* W1, int col) -> dash_status {
    Product p1 = prod(Xe, Xe, W0);
    p1.freeze = freeze;
    TRY(launch_gemm(&p1, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, Epilogue(), st));
    Product p2 = prod(W0, W0, W1);
    p2.freeze = freeze;
    TRY(launch_gemm(&p2, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, Epilogue(), st));
    Epilogue e;
    e.alpha = -0.25f;
    e.ia = CO_R1;
    e.gamma = 1.25f;
    e.coef = coef;
    e.monitor = res + col;
    e.mon_stride = 17;
    e.mon_mul = 16.f;
    Product p3 = prod(W1, A, Tout);
    p3.freeze = freeze;
    TRY(launch_gemm(&p3, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, e, st));
    return DASH_OK;
  };
  float* Tx = R[2];  // T(X)
  if ((r = evaluate(X, Tx, R[0], R[1], 0)) != DASH_OK) return r;
  for (int q = 0; q < refine; ++q) {
    float* Wc = R[0];  // candidate X T(X), then its symmetrised form in Xc
    float* Xc = R[1];
    Product p4 = prod(X, Tx, Wc);
    p4.freeze = freeze;
    TRY(launch_gemm(&p4, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, Epilogue(), st));
    Affine sym;
    sym.X = Wc;
    sym.D = Xc;
    sym.a = 1.f;
    TRY(launch_sym_affine(sym, N, B, st));
    // T of the candidate: X_c^2 into R[0] (free again), X_c^4 into the old T(X), T(X_c) into R[0]
    if ((r = evaluate(Xc, Wc, Wc, Tx, q + 1)) != DASH_OK) return r;
    TRY(launch_accept(res, 17, q, freeze, accept, Xc, X, N, B, st));
    // the accepted blocks' T is now in R[0]; the next step reads T from there
    std::swap(R[0], R[2]);
    Tx = R[2];
  }
  Affine fin;  // X = s^{-1/4} X, finite check (status bit 1)
  fin.X = X;
  fin.D = X;
  fin.a = 1.f;
  fin.ia = CO_U;
  fin.coef = coef;
  fin.status = status;
  TRY(launch_affine(fin, N, B, st));
  return DASH_OK;
}

}  // namespace

extern "C" {

dash_status dash_inverse_root_ndb_half(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, int32_t refine, float* X, float* monitor, int32_t* status,
                                       void* ws, size_t ws_bytes, void* stream) {
  return ndb_lowp_impl(A, s, N, B, iters1, iters2, DASH_FP16, refine, X, monitor, status, ws, ws_bytes, stream);
}

dash_status dash_inverse_root_ndb_lowp(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, dash_prec prec, int32_t refine, float* X, float* monitor,
                                       int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return ndb_lowp_impl(A, s, N, B, iters1, iters2, prec, refine, X, monitor, status, ws, ws_bytes, stream);
}

dash_status dash_inverse_root_ndb(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                  int32_t iters2, float* X, float* sqrt_out, float* monitor, int32_t* status,
                                  void* ws, size_t ws_bytes, void* stream) {
  return ndb_impl(A, s, N, B, iters1, iters2, X, sqrt_out, monitor, status, ws, ws_bytes, stream, Stop());
}

dash_status dash_inverse_root_ndb_prec(const float* A, const float* s, int64_t N, int32_t B, int32_t iters1,
                                       int32_t iters2, dash_prec prec, float* X, float* sqrt_out, float* monitor,
                                       int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return ndb_impl(A, s, N, B, iters1, iters2, X, sqrt_out, monitor, status, ws, ws_bytes, stream, Stop(), prec);
}

dash_status dash_inverse_root_ndb_adaptive(const float* A, const float* s, int64_t N, int32_t B, int32_t max_iters1,
                                           int32_t max_iters2, float tol, float* X, float* sqrt_out, float* monitor,
                                           int32_t* steps, int32_t* status, void* ws, size_t ws_bytes,
                                           void* stream) {
  if (!monitor || !(tol >= 0.f && tol < INFINITY) || (steps && !aligned(steps, 4))) return DASH_ERR_INVALID_ARG;
  Stop stop;
  stop.tol = tol;
  stop.steps = steps;
  return ndb_impl(A, s, N, B, max_iters1, max_iters2, X, sqrt_out, monitor, status, ws, ws_bytes, stream, stop);
}

}  // extern "C"

namespace {

dash_status cn_impl(const float* A, const float* s, int64_t N, int32_t B, int32_t p, int32_t iters, dash_prec prec,
                    float* X, float* monitor, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                    const Stop& stop) {
  if (!A || !s || !X || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (X == A || iters < 1 || iters > 1000) return DASH_ERR_INVALID_ARG;
  if (!fp32_prec(prec) && !half_prec(prec)) return DASH_ERR_INVALID_ARG;
  // split products: fp32 storage, products on the bfloat16 matrix cores where the shape allows
  const bool split = prec == DASH_FP32_SPLIT;
  if (split) prec = DASH_FP32;
  if (monitor && !aligned(monitor, 4)) return DASH_ERR_INVALID_ARG;
  if (status && !aligned(status, 4)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (p != 4) return DASH_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_cn(N, B, prec)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* coef = (float*)cv.take(coef_bytes(N));
  int32_t* freeze = (int32_t*)cv.take(flag_bytes(N));
  Pool pool;
  for (int q = 0; q < 5; ++q) pool.put(cv.take(stack_bytes(N, B, prec)));
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  if (monitor) TRY(launch_fill_f32(monitor, N * iters, 0.f, st));
  TRY(launch_coef(s, N, coef, status, st));
  const int T = iters;
  // adaptive stopping: a block whose monitor ||M_k - I|| is <= tol before step k >= 1 keeps X_k
  // from then on
  if (stop.freeze_ext) {
    if (T < 2 || stop.tol < 0.f || stop.steps || half_prec(prec)) return DASH_ERR_INVALID_ARG;
    freeze = stop.freeze_ext;
  } else if (stop.tol >= 0.f) {
    TRY(launch_freeze_reset(freeze, stop.steps, 1, T, N, st));
  } else {
    freeze = nullptr;
  }
  // binary16 (T >= 2, cn_half): triangle-only products, the iterates being symmetric polynomials
  // in A and the error floor set by binary16 storage; fp32 (below): full products, which keep the
  // fp32 rounding floor of the iteration lowest at high condition numbers
  // step 0: M_0 = A/s, S_0 = (5I - M_0)/4, X_1 = S_0;  ||M_0 - I||^2 = 16 ||S_0 - I||^2
  void* S = pool.get();
  void* M = pool.get();
  if (half_prec(prec) && T > 1) {  // 2-byte iterates: M_0 only; the S_k are formed inside the products
    pool.put(S);
    Affine m0;
    m0.X = A;
    m0.D = M;
    m0.d_prec = prec;
    m0.a = 1.f;
    m0.ia = CO_R1;
    m0.coef = coef;
    if (monitor) {
      m0.monitor = monitor;
      m0.mon_stride = T;
    }
    // built from the upper triangle of A: every later right operand is then exactly symmetric
    TRY(launch_sym_affine(m0, N, B, st));
    return cn_half(prec, N, B, T, X, monitor, status, coef, M, pool, st, freeze, stop.tol, stop.steps);
  }
  {
    Affine s0;
    s0.X = A;
    s0.D = S;
    s0.d_prec = prec;
    s0.a = -0.25f;
    s0.ia = CO_R1;
    s0.g = 1.25f;
    s0.coef = coef;
    if (T > 1) {
      s0.D2 = M;
      s0.d2_prec = prec;
      s0.a2 = 1.f;
      s0.ia2 = CO_R1;
    }
    if (monitor) {
      s0.monitor = monitor;
      s0.mon_stride = T;
      s0.mon_mul = 16.f;
    }
    // built from the upper triangle of A: every later right operand is then exactly symmetric
    TRY(launch_sym_affine(s0, N, B, st));
  }
  if (T == 1) {  // X = s^{-1/4} S_0, straight from A
    Affine fin;
    fin.X = A;
    fin.D = X;
    fin.a = -0.25f;
    fin.ia = CO_R1U;
    fin.g = 1.25f;
    fin.ig = CO_U;
    fin.coef = coef;
    TRY(launch_sym_affine(fin, N, B, st));
    Affine chk;  // finite check of the output (status bit 1)
    chk.X = X;
    chk.D = X;
    chk.a = 1.f;
    chk.status = status;
    if (status) TRY(launch_affine(chk, N, B, st));
    if (monitor) TRY(launch_monitor_finish(monitor, N * T, B, st));
    return DASH_OK;
  }
  // the fp32 products' arithmetic: the M S^4 launch that also writes S_{k+1} (a second output)
  // stays on the fp32 cores, as do stopped blocks
  const dash_prec pp = (split && B % 256 == 0 && !freeze) ? DASH_FP32_SPLIT : DASH_FP32;
  void* Xk = S;  // X_1 = S_0 shares the buffer (both are read-only from here on)
  for (int k = 0; k < T; ++k) {
    if (freeze && k >= 1)  // monitor column k (||M_k - I||) is complete
      TRY(launch_freeze_update(monitor, T, k, B, stop.tol, freeze, stop.steps, 1, k, N, st));
    if (k == T - 1) {  // X_T = s^{-1/4} X_{T-1} S_{T-1}
      Epilogue e;
      e.ia = CO_U;
      e.coef = coef;
      e.status = status;
      Product pr = prod(Xk, S, X);
      pr.freeze = freeze;
      pr.pass = 1;
      TRY(launch_gemm(&pr, 1, N, B, pp, DASH_FP32, Trans::NN, false, e, st, true));
      break;
    }
    void* S2 = pool.get();
    if (k == 0) {  // X_1 = S_0 needs no product; S_0 stays alive as X_1
      Product pr = prod(S, S, S2);
      pr.freeze = stop.freeze_ext;  // blocks left to another solver are skipped from the start
      TRY(launch_gemm(&pr, 1, N, B, pp, prec, Trans::NN, false, Epilogue(), st, true));
    } else {  // X_{k+1} = X_k S and S^2 in one launch; X_k and S are dead afterwards
      void* Xn = pool.get();
      Product pr[2] = {prod(Xk, S, Xn), prod(S, S, S2)};
      pr[0].freeze = pr[1].freeze = freeze;
      pr[0].pass = 1;  // a stopped block keeps X_k and needs no S^2
      TRY(launch_gemm(pr, 2, N, B, pp, prec, Trans::NN, false, Epilogue(), st, true));
      pool.put(Xk);
      pool.put(S);
      Xk = Xn;
    }
    void* S4 = pool.get();
    {
      Product pr = prod(S2, S2, S4);
      pr.freeze = freeze;
      TRY(launch_gemm(&pr, 1, N, B, pp, prec, Trans::NN, false, Epilogue(), st, true));
    }
    pool.put(S2);
    // M_{k+1} = M_k S^4 and S_{k+1} = (5I - M_{k+1})/4 from the same accumulator
    void* Sn = pool.get();
    Epilogue e;
    if (monitor) {
      e.monitor = monitor + (k + 1);
      e.mon_stride = T;
    }
    if (k + 1 == T - 1) {  // M_T is never needed: write S only, monitor from it
      e.alpha = -0.25f;
      e.gamma = 1.25f;
      e.mon_mul = 16.f;
      Product pr = prod(M, S4, Sn);
      pr.freeze = freeze;
      TRY(launch_gemm(&pr, 1, N, B, pp, prec, Trans::NN, false, e, st, true));
      pool.put(M);
      M = nullptr;
    } else {
      void* Mn = pool.get();
      e.alpha = 1.f;
      e.alpha2 = -0.25f;
      e.gamma2 = 1.25f;
      Product pr = prod(M, S4, Mn, nullptr, nullptr, Sn);
      pr.freeze = freeze;
      TRY(launch_gemm(&pr, 1, N, B, prec, prec, Trans::NN, false, e, st, true));
      pool.put(M);
      M = Mn;
    }
    pool.put(S4);
    S = Sn;
  }
  if (monitor) TRY(launch_monitor_finish(monitor, N * T, B, st));
  return DASH_OK;
}

}  // namespace

extern "C" {

dash_status dash_inverse_root_cn(const float* A, const float* s, int64_t N, int32_t B, int32_t p, int32_t iters,
                                 dash_prec prec, float* X, float* monitor, int32_t* status, void* ws,
                                 size_t ws_bytes, void* stream) {
  return cn_impl(A, s, N, B, p, iters, prec, X, monitor, status, ws, ws_bytes, stream, Stop());
}

dash_status dash_inverse_root_cn_adaptive(const float* A, const float* s, int64_t N, int32_t B, int32_t p,
                                          int32_t max_iters, float tol, dash_prec prec, float* X, float* monitor,
                                          int32_t* steps, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (!monitor || !(tol >= 0.f && tol < INFINITY) || (steps && !aligned(steps, 4))) return DASH_ERR_INVALID_ARG;
  Stop stop;
  stop.tol = tol;
  stop.steps = steps;
  return cn_impl(A, s, N, B, p, max_iters, prec, X, monitor, status, ws, ws_bytes, stream, stop);
}

dash_status dash_inverse_root_cheb(const float* A, const float* s, int64_t N, int32_t B, int32_t degree, double lo,
                                   double hi, float* X, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return dash_inverse_root_cheb_prec(A, s, N, B, degree, lo, hi, DASH_FP32, X, status, ws, ws_bytes, stream);
}

dash_status dash_inverse_root_cheb_prec(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                        double lo, double hi, dash_prec prec, float* X, int32_t* status, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (!(std::isfinite(lo) && std::isfinite(hi) && lo > 0.0 && hi > lo)) return DASH_ERR_INVALID_ARG;
  ChebInterval iv;
  iv.lo_rel = lo;
  iv.hi = hi;
  return cheb_impl(A, s, N, B, degree, iv, prec, X, nullptr, status, ws, ws_bytes, stream);
}

dash_status dash_inverse_root_cheb_blocks(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                          double floor, const float* lam_min, float theta, double hi, dash_prec prec,
                                          float* X, float* lo_out, int32_t* status, void* ws, size_t ws_bytes,
                                          void* stream) {
  if (!(std::isfinite(floor) && floor >= 0.0 && std::isfinite(hi) && hi > 0.0)) return DASH_ERR_INVALID_ARG;
  if (lam_min && (!aligned(lam_min, 4) || !(theta > 0.f && theta <= 1.f))) return DASH_ERR_INVALID_ARG;
  if (!lam_min && !(floor > 0.0)) return DASH_ERR_INVALID_ARG;
  ChebInterval iv;
  iv.floor = floor;
  iv.lam = lam_min;
  iv.theta = theta;
  iv.hi = hi;
  return cheb_impl(A, s, N, B, degree, iv, prec, X, lo_out, status, ws, ws_bytes, stream);
}

dash_status dash_inverse_root_evd(const float* A, int64_t N, int32_t B, int32_t max_sweeps, int32_t refine, float* X,
                                  float* eigvals, int32_t* sweeps, int32_t* status, void* ws, size_t ws_bytes,
                                  void* stream) {
  return dash_inverse_root_evd_prec(A, N, B, max_sweeps, refine, DASH_FP32, X, eigvals, sweeps, status, ws, ws_bytes,
                                    stream);
}

dash_status dash_inverse_root_evd_prec(const float* A, int64_t N, int32_t B, int32_t max_sweeps, int32_t refine,
                                       dash_prec prec, float* X, float* eigvals, int32_t* sweeps, int32_t* status,
                                       void* ws, size_t ws_bytes, void* stream) {
  if (!A || !X || A == X || !aligned(A, 16) || !aligned(X, 16) || !valid_N(N)) return DASH_ERR_INVALID_ARG;
  if (max_sweeps < 1 || max_sweeps > 100 || (refine != 0 && refine != 1)) return DASH_ERR_INVALID_ARG;
  // the binary16 pass only finds the eigenvectors approximately; the fp32 pass must follow it
  if (prec != DASH_FP32 && !(prec == DASH_FP16 && refine == 1)) return DASH_ERR_INVALID_ARG;
  const bool half = prec == DASH_FP16;
  if ((eigvals && !aligned(eigvals, 4)) || (sweeps && !aligned(sweeps, 4)) || (status && !aligned(status, 4)))
    return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_evd(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* V = (float*)cv.take((size_t)N * B * B * sizeof(float));
  float* T = (float*)cv.take((size_t)N * B * B * sizeof(float));
  JacobiPlan jp;
  jp.N = N;
  jp.B = B;
  jp.max_sweeps = max_sweeps;
  jp.pass = 0;
  jp.tol = 0x1p-22f;
  jp.R = (float*)cv.take((size_t)N * (B / 64) * 64 * 64 * sizeof(float));
  jp.rot = (int32_t*)cv.take((size_t)N * (B / 64) * sizeof(int32_t));
  float* scale = (float*)cv.take((size_t)N * B * sizeof(float));
  jp.flags = (int32_t*)cv.take((size_t)N * 8 * sizeof(int32_t));
  float* coef = (float*)cv.take((size_t)N * COEF_STRIDE * sizeof(float));
  jp.rsc = (float*)cv.take((size_t)N * (B / 64) * sizeof(float));
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  // pass 1 on a working copy of A held in X, eigenvectors accumulated in V
  TRY(hipMemcpyAsync(X, A, (size_t)N * B * B * sizeof(float), hipMemcpyDeviceToDevice, st));
  TRY(launch_identity(V, N, B, st));
  jp.A = X;
  jp.V = V;
  // a first pass that the refinement pass follows finds the eigenvectors only approximately: its
  // pair sub-problems run in fp32 (the refinement pass forms H from A again and runs fp64 ones)
  jp.pair_f32 = refine == 1;
  if (half) {
    // pass 1 with fp32 pair sub-problems; rotations below binary16's resolution are left to the
    // refinement pass, which removes the binary16 rounding of the dense sweeps
    // the dense working matrix's eigenvalues reach up to B times its largest diagonal entry: that
    // entry maps to at most 1
    TRY(launch_half_prescale(A, N, B, coef, st));
    jp.half = true;
    jp.coef = coef;
    jp.tol = 0x1p-11f;
  }
  TRY(launch_jacobi(jp, st));
  // pass 2 (if any) in fp32 throughout: its rotations between nearly equal eigenvalues are not small
  // even when H is nearly diagonal, so binary16 corrections would cost the eigenvectors accuracy
  jp.half = false;
  jp.pair_f32 = false;
  jp.tol = 0x1p-22f;
  EvdFinish fin;
  fin.N = N;
  fin.B = B;
  fin.scale = scale;
  fin.flags = jp.flags;
  fin.eigvals = eigvals;
  fin.sweeps = sweeps;
  fin.status = status;
  if (refine) {
    // Newton-Schulz steps Q <- Q (3I - Q^T Q) / 2 on the eigenvector estimate (one after the fp32
    // pass; two after the binary16 pass, whose estimate is orthogonal only to about 1e-2), then
    // H = Q^T (A Q) from the input A; pass 2 diagonalises H in T and rotates Q
    Epilogue ns;
    ns.alpha = -0.5f;
    ns.gamma = 1.5f;
    float* Q = V;     // current estimate
    float* free = X;  // the working copy of pass 1 is no longer needed
    for (int it = 0; it < (half ? 2 : 1); ++it) {
      Product p1 = prod(Q, Q, T);
      TRY(launch_gemm(&p1, 1, N, B, DASH_FP32, DASH_FP32, Trans::TN, true, ns, st));
      Product p2 = prod(Q, T, free);
      TRY(launch_gemm(&p2, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, Epilogue(), st));
      float* tmp = Q;
      Q = free;
      free = tmp;
    }
    Product p3 = prod(A, Q, free);
    TRY(launch_gemm(&p3, 1, N, B, DASH_FP32, DASH_FP32, Trans::NN, false, Epilogue(), st));
    Product p4 = prod(Q, free, T);
    TRY(launch_gemm(&p4, 1, N, B, DASH_FP32, DASH_FP32, Trans::TN, true, Epilogue(), st));
    jp.pass = 1;
    jp.A = T;
    jp.V = Q;
    TRY(launch_jacobi(jp, st));
    fin.A = T;
    fin.V = Q;
    // Y = Q diag(w^-1/8) must not be X, the output of the last product
    fin.Y = Q == X ? free : Q;
  } else {
    fin.A = X;
    fin.V = V;
    fin.Y = V;
  }
  TRY(launch_evd_finish(fin, st));
  Epilogue e;  // X = Y Y^T, Y = V diag(w^{-1/8}); finite check of the output (status bit 1)
  e.status = status;
  Product pr = prod(fin.Y, fin.Y, X);
  TRY(launch_gemm(&pr, 1, N, B, DASH_FP32, DASH_FP32, Trans::NT, true, e, st));
  return DASH_OK;
}

dash_status dash_apply(const float* XL, const float* XR, const float* G_stack, int64_t NG, int32_t B, float* U_stack,
                       void* ws, size_t ws_bytes, void* stream) {
  return dash_apply_prec(XL, XR, G_stack, NG, B, DASH_FP32, U_stack, ws, ws_bytes, stream);
}

dash_status dash_apply_prec(const float* XL, const float* XR, const float* G_stack, int64_t NG, int32_t B,
                            dash_prec prec, float* U_stack, void* ws, size_t ws_bytes, void* stream) {
  if (!fp32_prec(prec) && prec != DASH_FP32_SPLIT16) return DASH_ERR_INVALID_ARG;
  if (!XL || !XR || !G_stack || !U_stack || !valid_N(NG)) return DASH_ERR_INVALID_ARG;
  if (!aligned(XL, 16) || !aligned(XR, 16) || !aligned(G_stack, 16) || !aligned(U_stack, 16))
    return DASH_ERR_INVALID_ARG;
  if (U_stack == XL || U_stack == XR || U_stack == G_stack) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_apply(NG, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* T = (float*)cv.take(stack_bytes(NG, B, DASH_FP32));
  const bool h2 = prec == DASH_FP32_SPLIT16 && B % 256 == 0;
  const dash_prec pp = h2 ? DASH_FP32_SPLIT16
                          : ((prec == DASH_FP32_SPLIT || prec == DASH_FP32_SPLIT16) && B % 256 == 0) ? DASH_FP32_SPLIT
                                                                                                       : DASH_FP32;
  Product p1 = prod(XL, G_stack, T);
  Product p2 = prod(T, XR, U_stack);
  if (h2) {  // two-piece binary16: passes over XL, G and XR; T's bound from the first launch
    float* b[3];
    for (int i = 0; i < 3; ++i) b[i] = (float*)cv.take(align_up((size_t)NG * sizeof(float), 256));
    float* bt = (float*)cv.take(align_up((size_t)NG * ndb_parts(B) * sizeof(float), 256));
    TRY(launch_block_amax(XL, NG, B, b[0], st));
    TRY(launch_block_amax(G_stack, NG, B, b[1], st));
    TRY(launch_block_amax(XR, NG, B, b[2], st));
    p1.amax_x = b[0];
    p1.amax_y = b[1];
    p1.amax_d = bt;
    p2.amax_x = bt;
    p2.amax_x_parts = (int)ndb_parts(B);
    p2.amax_y = b[2];
  }
  TRY(launch_gemm(&p1, 1, NG, B, pp, DASH_FP32, Trans::NN, false, Epilogue(), st));
  TRY(launch_gemm(&p2, 1, NG, B, pp, DASH_FP32, Trans::NN, false, Epilogue(), st));
  return DASH_OK;
}

// ------------------------------------------------------------------------------------------------
// Spectrum bounds, the residual probe and the routed (two-solver) inverse root
// ------------------------------------------------------------------------------------------------

dash_status dash_spectrum_min(const float* A, const float* s, int64_t N, int32_t B, double hi, int32_t k,
                              int32_t steps, const float* V0, float* lam_min, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!A || !s || !V0 || !lam_min || !aligned(A, 16) || !aligned(s, 4) || !aligned(V0, 4) || !aligned(lam_min, 4) ||
      !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (!(std::isfinite(hi) && hi > 0.0) || k < 1 || k > 32 || steps < 1 || steps > 10000) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < power_workspace_bytes(N, B, DASH_FP32)) return DASH_ERR_WORKSPACE;
  Carver cv{(char*)ws, ws_bytes};
  PowerPlan p;
  p.N = N;
  p.B = B;
  p.k = k;
  p.steps = steps;
  p.prec = DASH_FP32;
  p.A = A;
  p.V0 = V0;
  p.s = lam_min;
  const int RB = B / 64;
  for (int q = 0; q < 2; ++q) p.W[q] = (float*)cv.take((size_t)N * B * 32 * sizeof(float));
  for (int q = 0; q < 2; ++q) p.part[q] = (float*)cv.take((size_t)N * RB * 3 * 32 * sizeof(float));
  p.V0p = (float*)cv.take((size_t)B * 32 * sizeof(float));
  p.coef = (float*)cv.take((size_t)N * COEF_STRIDE * sizeof(float));
  p.Ah = nullptr;
  p.shift_s = s;
  p.shift_mul = (float)hi;
  TRY(launch_power_iteration(p, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_residual_probe(const float* A, const float* X, int64_t N, int32_t B, int32_t k, const float* V0,
                                float* r, void* ws, size_t ws_bytes, void* stream) {
  if (!A || !X || !V0 || !r || !aligned(A, 16) || !aligned(X, 16) || !aligned(V0, 4) || !aligned(r, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (k < 1 || k > 32) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < power_workspace_bytes(N, B, DASH_FP32)) return DASH_ERR_WORKSPACE;
  Carver cv{(char*)ws, ws_bytes};
  ProbePlan p;
  p.N = N;
  p.B = B;
  p.k = k;
  p.A = A;
  p.X = X;
  p.V0 = V0;
  p.r = r;
  const int RB = B / 64;
  for (int q = 0; q < 2; ++q) p.W[q] = (float*)cv.take((size_t)N * B * 32 * sizeof(float));
  for (int q = 0; q < 2; ++q) p.part[q] = (float*)cv.take((size_t)N * RB * 3 * 32 * sizeof(float));
  p.V0p = (float*)cv.take((size_t)B * 32 * sizeof(float));
  TRY(launch_residual_probe(p, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_inverse_root_routed(const float* A, const float* s, int64_t N, int32_t B, int32_t degree,
                                     double floor, double hi, int32_t k, int32_t est_steps, const float* V0,
                                     float tol, int32_t cn_iters, dash_prec prec, float* X, float* lam_min,
                                     float* resid, int32_t* route, int32_t* status, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!fp32_prec(prec) && prec != DASH_FP32_SPLIT16) return DASH_ERR_INVALID_ARG;
  if (!A || !s || !X || !V0 || X == A || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !aligned(V0, 4) ||
      !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if ((lam_min && !aligned(lam_min, 4)) || (resid && !aligned(resid, 4)) || (route && !aligned(route, 4)) ||
      (status && !aligned(status, 4)))
    return DASH_ERR_INVALID_ARG;
  if (degree < 1 || degree > CHEB_MAX_DEGREE || !(std::isfinite(floor) && floor >= 0.0) ||
      !(std::isfinite(hi) && hi > 0.0) || k < 1 || k > 32 || est_steps < 0 || est_steps > 10000 ||
      !(tol > 0.f && tol < INFINITY) || cn_iters < 2 || cn_iters > ROUTED_MAX_CN_ITERS)
    return DASH_ERR_INVALID_ARG;
  if (est_steps == 0 && !(floor > 0.0)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_routed(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* lam = (float*)cv.take((size_t)N * sizeof(float));
  float* r = (float*)cv.take((size_t)N * sizeof(float));
  int32_t* rt = (int32_t*)cv.take(flag_bytes(N));
  if (lam_min) lam = lam_min;
  if (route) rt = route;
  int32_t* freeze = (int32_t*)cv.take(flag_bytes(N));
  int32_t* cn_status = (int32_t*)cv.take(flag_bytes(N));
  float* monitor = (float*)cv.take((size_t)N * ROUTED_MAX_CN_ITERS * sizeof(float));
  void* region = cv.p;
  const size_t region_bytes = cv.left;
  dash_status rc;
  // 1. the smallest eigenvalue of every block, estimated from above by the shifted power iteration
  if (est_steps > 0) {
    rc = dash_spectrum_min(A, s, N, B, hi, k, est_steps, V0, lam, region, region_bytes, stream);
    if (rc != DASH_OK) return rc;
  }
  // 2. Chebyshev on [max(floor, lam/2)/s, hi] per block
  ChebInterval iv;
  iv.floor = floor;
  iv.lam = est_steps > 0 ? lam : nullptr;
  iv.theta = 0.5f;
  iv.hi = hi;
  rc = cheb_impl(A, s, N, B, degree, iv, prec, X, nullptr, status, region, region_bytes, stream);
  if (rc != DASH_OK) return rc;
  // 3. its residual per block, by the probe; 4. blocks above tol (or NaN) go to coupled Newton
  rc = dash_residual_probe(A, X, N, B, k, V0, r, region, region_bytes, stream);
  if (rc != DASH_OK) return rc;
  TRY(launch_route(r, tol, N, rt, freeze, st));
  // 5. coupled Newton p = 4 (fp32 cores) on the routed blocks only, each stopping once its residual
  // ||M_k - I|| / sqrt(B) is <= tol / 2; the other blocks' X is left as the Chebyshev solve wrote it
  Stop stop;
  stop.tol = 0.5f * tol;
  stop.freeze_ext = freeze;
  rc = cn_impl(A, s, N, B, 4, cn_iters, DASH_FP32, X, monitor, cn_status, region, region_bytes, stream, stop);
  if (rc != DASH_OK) return rc;
  if (status) TRY(launch_select_i32(cn_status, rt, status, N, st));
  if (lam_min && est_steps == 0) TRY(launch_fill_f32(lam_min, N, __builtin_nanf(""), st));
  // 6. the final residual of every block, by the probe
  if (resid) {
    rc = dash_residual_probe(A, X, N, B, k, V0, resid, region, region_bytes, stream);
    if (rc != DASH_OK) return rc;
  }
  return DASH_OK;
}

// ------------------------------------------------------------------------------------------------
// 1-D parameters
// ------------------------------------------------------------------------------------------------

static dash_status check_vecs(const dash_vec* v, int32_t n, int32_t B) {
  if (!v || n < 1) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i)
    if (!v[i].ptr || !aligned(v[i].ptr, 4) || v[i].len < 1) return DASH_ERR_INVALID_ARG;
  return DASH_OK;
}

dash_status dash_stack_vec(const dash_vec* grads, int32_t n, int32_t B, float* g_pieces, void* stream) {
  const dash_status chk = check_vecs(grads, n, B);
  if (chk != DASH_OK) return chk;
  if (!g_pieces || !aligned(g_pieces, 4)) return DASH_ERR_INVALID_ARG;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    TRY(launch_vec_copy(grads[i].ptr, grads[i].len, g_pieces + off, B, true, as_stream(stream)));
    off += (grads[i].len + B - 1) / B * B;
  }
  return DASH_OK;
}

dash_status dash_unstack_vec(const float* u_pieces, int32_t B, const dash_vec* outs, int32_t n, void* stream) {
  const dash_status chk = check_vecs(outs, n, B);
  if (chk != DASH_OK) return chk;
  if (!u_pieces || !aligned(u_pieces, 4)) return DASH_ERR_INVALID_ARG;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    TRY(launch_vec_copy(outs[i].ptr, outs[i].len, (float*)u_pieces + off, B, false, as_stream(stream)));
    off += (outs[i].len + B - 1) / B * B;
  }
  return DASH_OK;
}

dash_status dash_update_stats_vec(const float* g_pieces, int64_t P, int32_t B, float beta, float* L, void* stream) {
  if (!g_pieces || !L || !aligned(g_pieces, 16) || !aligned(L, 16) || !valid_N(P)) return DASH_ERR_INVALID_ARG;
  if (!(beta >= 0.f && beta <= 1.f)) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  TRY(launch_vec_stats(g_pieces, P, B, beta, L, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_apply_vec(const float* X, const float* g_pieces, int64_t P, int32_t B, float* u_pieces, void* stream) {
  if (!X || !g_pieces || !u_pieces || !aligned(X, 16) || !aligned(g_pieces, 16) || !aligned(u_pieces, 4) ||
      !valid_N(P) || u_pieces == g_pieces)
    return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  TRY(launch_vec_apply(X, g_pieces, P, B, u_pieces, as_stream(stream)));
  return DASH_OK;
}

dash_status dash_inverse_sqrt_ndb(const float* A, const float* s, int64_t N, int32_t B, int32_t iters, dash_prec prec,
                                  float* X, float* monitor, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (!fp32_prec(prec)) return DASH_ERR_INVALID_ARG;
  if (!A || !s || !X || !aligned(A, 16) || !aligned(X, 16) || !aligned(s, 4) || !valid_N(N))
    return DASH_ERR_INVALID_ARG;
  if (X == A || iters < 1 || iters > 1000) return DASH_ERR_INVALID_ARG;
  if ((monitor && !aligned(monitor, 4)) || (status && !aligned(status, 4))) return DASH_ERR_INVALID_ARG;
  if (!valid_B(B)) return DASH_ERR_SHAPE;
  if (!ws || !aligned(ws, 256) || ws_bytes < ws_ndb(N, B)) return DASH_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  Carver cv{(char*)ws, ws_bytes};
  float* coef = (float*)cv.take(coef_bytes(N));
  (void)cv.take(flag_bytes(N));
  Pool pool;
  for (int q = 0; q < 5; ++q) pool.put(cv.take(stack_bytes(N, B, DASH_FP32)));
  if (status) TRY(launch_fill_i32(status, N, 0, st));
  if (monitor) TRY(launch_fill_f32(monitor, N * iters, 0.f, st));
  TRY(launch_coef(s, N, coef, status, st));
  NdbCtx c{N, B, coef, monitor, iters, status, st, &pool};
  c.split = prec == DASH_FP32_SPLIT;
  c.final_ia = CO_RSQ;  // X = s^{-1/2} Z
  const dash_status r = ndb_call(c, A, false, true, iters, 0, true, X, nullptr);
  if (r != DASH_OK) return r;
  if (monitor) TRY(launch_monitor_finish(monitor, N * iters, B, st));
  return DASH_OK;
}

}  // extern "C"
