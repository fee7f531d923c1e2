// cheb.hip -- the per-block Chebyshev/Clenshaw plan and the routing helpers of the two-solver call.
//
// The Chebyshev solver ([PT] Metodologia, item 2, "Aproximações de Polinômios de Chebyshev")
// evaluates on A_b / s_b the degree-d interpolant of x^{-1/4} at the d+1 Chebyshev points of the
// first kind of an interval [lo_b, hi].  The plan kernel derives, per block and on the device, the
// interval (from s_b, a floor and an optional per-block lower estimate), the interpolation
// coefficients in fp64, and the epilogue coefficients of every product launch of the Clenshaw
// recurrence, so a stack whose blocks differ in scale or conditioning gets an interval of its own
// per block without the host reading s.
#include <hip/hip_runtime.h>

#include <cmath>

#include "dash_internal.hpp"

namespace dash {
namespace {

// One 64-thread workgroup per block.
__global__ __launch_bounds__(64) void cheb_plan_kernel(ChebPlan p) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = p.d;
  __shared__ double fx[CHEB_MAX_DEGREE + 1], c[CHEB_MAX_DEGREE + 1];
  __shared__ double lo_sh;
  __shared__ int bad;
  if (tid == 0) {
    double lo;
    if (p.lo_rel > 0.0) {
      lo = p.lo_rel;
    } else {
      double f = p.floor;
      if (p.lam) {
        const double l = (double)p.theta * (double)p.lam[b];
        if (l > f) f = l;  // a NaN estimate leaves the floor
      }
      lo = f / (double)p.s[b];
    }
    lo_sh = lo;
    bad = !(isfinite(lo) && lo > 0.0 && lo < p.hi);
  }
  __syncthreads();
  const double lo = lo_sh, hi = p.hi, w = hi - lo, m = hi + lo;
  const double pi = 3.14159265358979323846;
  // interpolation at x_j = ((hi - lo) cos(theta_j) + hi + lo) / 2, theta_j = pi (j + 1/2) / (d + 1)
  for (int j = tid; j <= d; j += 64) {
    const double th = pi * (j + 0.5) / (d + 1);
    const double x = 0.5 * ((hi - lo) * cos(th) + hi + lo);
    fx[j] = 1.0 / sqrt(sqrt(x));
  }
  __syncthreads();
  for (int k = tid; k <= d; k += 64) {
    double acc = 0.0;
    for (int j = 0; j <= d; ++j) acc += fx[j] * cos(k * (pi * (j + 0.5) / (d + 1)));
    acc *= 2.0 / (d + 1);
    c[k] = k == 0 ? 0.5 * acc : acc;
  }
  __syncthreads();

  const float* cf = p.coef + b * COEF_STRIDE;
  const float R1 = cf[CO_R1], R2 = cf[CO_R2], U = cf[CO_U], S = cf[CO_S], R1U = cf[CO_R1U];
  // b_d = c_d I and b_{d-1} = c_{d-1} I + 2 T b_d = a1 A/s + g1 I are never stored
  const double a1 = d >= 1 ? 4.0 * c[d] / w : 0.0;
  const double g1 = d >= 1 ? c[d - 1] - 2.0 * c[d] * m / w : 0.0;
  const int P = d == 1 ? 1 : d - 1;
  for (int q = tid; q < P; q += 64) {
    float row[COEF_STRIDE] = {};
    bool ok = !bad;
    if (d == 1) {  // X = u (c0 I + c1 T), T = (2 A/s - (hi + lo) I) / (hi - lo)
      row[CS_ALPHA] = (float)(2.0 * c[1] / w) * R1U;
      row[CS_GAMMA] = (float)(c[0] - c[1] * m / w) * U;
    } else {
      // launch q forms b_k, k = d - 2 - q; the last one (k = 0) forms X = u (c_0 I + T b_1 - b_2)
      const int k = d - 2 - q;
      const bool last = (k == 0);
      // b_k = c_k I + 2 T b_{k+1} - b_{k+2} = alpha (A b_{k+1} + c_over_a b_{k+1}) + delta b_{k+2} + gamma I
      if (last) {
        row[CS_ALPHA] = (float)(2.0 / w) * R1U;
        row[CS_BETA] = (float)(-m / w) * U;
        row[CS_DELTA] = -1.f * U;
      } else {
        row[CS_ALPHA] = (float)(4.0 / w) * R1;
        row[CS_BETA] = (float)(-2.0 * m / w);
        row[CS_DELTA] = -1.f;
      }
      row[CS_COVERA] = (float)(-0.5 * m) * S;
      if (q == 0) {
        if (p.split_first) {
          // alpha A b_{d-1} + beta b_{d-1} + gamma I with b_{d-1} = a1 A/s + g1 I, as
          // (alpha a1 / s)(A + c I) A + (gamma + beta g1) I, c = s (g1/a1 - m/2); no b_{d+1} term
          ok = ok && a1 != 0.0;
          row[CS_ALPHA] = (float)(4.0 * a1 / w) * R2;
          row[CS_COVERA] = (float)(g1 / a1 - 0.5 * m) * S;
          row[CS_GAMMA] = (float)(c[d - 2] - c[d] - 2.0 * m / w * g1);
          row[CS_DELTA] = 0.f;
          ok = ok && row[CS_ALPHA] != 0.f;
        } else {  // the right operand A is read as b_{d-1} = a1 A/s + g1 I; b_{k+2} = b_d = c_d I
          row[CS_MAPA] = (float)a1 * R1;
          row[CS_MAPG] = (float)g1;
          row[CS_GAMMA] = (float)((last ? c[0] : c[d - 2]) - c[d]) * (last ? U : 1.f);
        }
      } else if (q == 1) {  // b_{k+2} = b_{d-1} = a1 A/s + g1 I, read as A with its coefficients
        row[CS_DELTA] = (float)(-a1) * (last ? R1U : R1);
        row[CS_GAMMA] = (float)((last ? c[0] : c[d - 3]) - g1) * (last ? U : 1.f);
      } else {
        row[CS_GAMMA] = last ? (float)c[0] * U : (float)c[k];
      }
    }
    for (int e = 0; e < COEF_STRIDE; ++e) ok = ok && isfinite(row[e]);
    if (!ok) {
      for (int e = 0; e < COEF_STRIDE; ++e) row[e] = __builtin_nanf("");
      if (p.status) atomicOr(&p.status[b], 1);
    }
    float* t = p.tab + ((int64_t)q * p.N + b) * COEF_STRIDE;
    for (int e = 0; e < COEF_STRIDE; ++e) t[e] = row[e];
  }
  if (tid == 0 && p.lo_out) p.lo_out[b] = bad ? __builtin_nanf("") : (float)lo;
}

__global__ void route_kernel(const float* r, float tol, int64_t N, int32_t* route, int32_t* freeze) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= N) return;
  const int32_t second = !(r[b] <= tol);  // NaN goes to the second solver
  route[b] = second;
  freeze[b] = second ? 0 : 2;
}

__global__ void select_i32_kernel(const int32_t* src, const int32_t* route, int32_t* dst, int64_t N) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b < N && route[b]) dst[b] = src[b];
}

}  // namespace

hipError_t launch_cheb_plan(const ChebPlan& p, hipStream_t stream) {
  if (p.N < 1 || p.N > 0x7fffffffLL || p.d < 1 || p.d > CHEB_MAX_DEGREE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cheb_plan_kernel, dim3((unsigned)p.N), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_route(const float* r, float tol, int64_t N, int32_t* route, int32_t* freeze, hipStream_t stream) {
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, r, tol, N, route, freeze);
  return hipGetLastError();
}

hipError_t launch_select_i32(const int32_t* src, const int32_t* route, int32_t* dst, int64_t N, hipStream_t stream) {
  hipLaunchKernelGGL(select_i32_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream, src, route, dst, N);
  return hipGetLastError();
}

}  // namespace dash
