// cat_noalloc.hip -- the 1D forward for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc): cat_forward_1d_noalloc takes no workspace argument and
// runs the kernels of cat_forward_1d on a fixed scratch array that the
// library holds in device memory.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy, at its own address, from module load until the
// process ends.  In host code its name is a host-side stand-in, not a device
// address: the first call on a device (with that device current) asks the
// runtime for that device's address with hipGetSymbolAddress and keeps it;
// every later use -- the kernels' workspace argument -- takes that address.
//
// The forward writes every scratch byte it reads (V, the logits and the
// spectrum, or the long path's intermediates) before reading it, so nothing
// needs clearing between calls.  All calls on one GPU share the array:
// calls that overlap on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/cat.h"
#include "cat_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(CAT_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

__device__ __attribute__((used)) __align__(256) static unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up once per device).
cat_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return cat::set_error(CAT_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return cat::set_error(CAT_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return cat::set_error(CAT_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return CAT_OK;
}

}  // namespace

extern "C" cat_status cat_forward_1d_noalloc(cat_plan plan, const void* X, const void* W_A, const void* W_V, void* O,
                                             void* stream) {
  cat_status st = cat::plan_check_forward_1d(plan, X, W_A, W_V, O);
  if (st != CAT_OK) return st;
  if (cat::plan_batch(plan) == 0) return CAT_OK;
  if (cat::plan_forward_ws_bytes(plan) > kScratchBytes)
    return cat::set_error(CAT_ERR_UNSUPPORTED,
                          "problem needs more scratch than the library's fixed array (CAT_NOALLOC_SCRATCH_BYTES)");
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != CAT_OK) return st;
  return cat::forward_1d_checked(plan, X, W_A, W_V, O, ws, stream);
}
