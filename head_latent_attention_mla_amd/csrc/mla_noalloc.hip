// Scratch memory of the allocation-free decode call (mla_decode_attn_noalloc).
//
// The split-T scan keeps its per-part partial outputs, log-sum-exps and the
// per-sequence part tables in a workspace.  For callers that cannot allocate
// (code under graph capture, serving loops, harnesses that forbid it), that
// workspace is a file-scope device array of fixed size instead.  In host code
// the array's name is only a stand-in for the symbol, not a device address:
// the address every kernel argument and copy must use is looked up once per
// device with hipGetSymbolAddress and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.h"

namespace mla {

namespace {

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    // with this device current (the caller's), once: the device address of
    // this device's copy of the array
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
