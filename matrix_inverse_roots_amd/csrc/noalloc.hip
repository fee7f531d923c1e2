// noalloc.hip -- dash_scale_noalloc: the per-block scale without a caller workspace, for callers that
// cannot allocate device memory (code under stream capture, tight serving loops).
//
// The power iteration's scratch (its two iterate buffers, their column partials, the prepared start
// vectors, the coefficient table and, for binary16, the cast of A) lives in one file-scope device
// array of SCRATCH_BYTES per GPU, held until the process ends.  Host code never uses the array's
// name as an address: the device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept.  Every call on a GPU shares that GPU's array and leaves its contents
// behind; nothing in it has to start at zero (every buffer is written before it is read).  Two calls
// that overlap on one GPU (e.g. on two streams) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dash_internal.hpp"

namespace dash {
namespace {

constexpr size_t SCRATCH_BYTES = size_t(128) << 20;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of `scratch` (looked up on the first call on that device), or null.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace
}  // namespace dash

extern "C" {

size_t dash_noalloc_scratch_bytes(void) { return dash::SCRATCH_BYTES; }

dash_status dash_scale_noalloc(const float* A, int64_t N, int32_t B, dash_scaling how, dash_prec prec, int32_t k,
                               int32_t steps, const float* V0, uint64_t seed, float* s, void* stream) {
  using namespace dash;
  const dash_status chk = scale_args_check(A, N, B, how, prec, k, steps, V0, s);
  if (chk != DASH_OK) return chk;
  if (how == DASH_SCALE_FROBENIUS) return dash_scale(A, N, B, how, prec, k, steps, V0, seed, s, nullptr, 0, stream);
  // the request must fit the fixed scratch; decided on the host before any device call
  if (power_workspace_bytes(N, B, prec) > SCRATCH_BYTES) return DASH_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return DASH_ERR_DEVICE;
  return dash_scale(A, N, B, how, prec, k, steps, V0, seed, s, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"
