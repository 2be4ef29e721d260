// Library-owned device scratch for the allocation-free forward entry point
// (lard_relkl_fwd_noalloc): the forward's per-workgroup fp64 loss partials, which the
// other entry points keep in the caller's workspace.  One array per GPU, held until the
// process ends; every call on a GPU shares it, so calls that overlap on one GPU race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "relkl_internal.h"

namespace lard {

static __device__ __align__(256) double scratch[kNoallocMaxPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and cached.  In host code the array's name is only a host-side stand-in:
// every use of the memory goes through this address.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return 0;
}

}  // namespace lard
