// Device scratch for the allocation-free entry point (sla_pool_classify_noalloc):
// a file-scope device array that takes the place of the caller's workspace.
// Each GPU the library runs on holds its own copy, at its own address, until
// the process ends.  Host code never passes the array's name to a kernel or a
// copy: the name is a host-side stand-in, and the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace sla {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sla
