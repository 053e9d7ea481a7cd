// Fixed device scratch for the allocation-free attention entry point (hstu_attn_fwd_noalloc).
//
// The scratch of hstu_attn_fwd -- the per-32-token timestamp ranges its prologue kernel writes and
// its attention kernel reads -- lives here in a file-scope device array instead of a caller
// workspace, so that callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops) can run the forward with only their inputs and outputs.  Every GPU holds its own
// copy of the array from the library's load until the process ends.  In host code the array's name
// is only a host-side handle: its device address is looked up once per device (with that device
// current) through hipGetSymbolAddress and kept, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace hstu {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  if (!g_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace hstu
