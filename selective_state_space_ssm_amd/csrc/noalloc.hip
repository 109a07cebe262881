// Fixed device scratch for the entry point that allocates nothing
// (ssm_scan_fwd_noalloc): the two-pass plan's chunk aggregates and chunk
// start states live in a file-scope device array instead of a
// stream-ordered allocation.
//
// Every GPU the library runs on holds its own copy of `scratch` until the
// process ends.  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels.  Calls that overlap on one GPU share the array and
// race; the kernels write every word of it they read within one call, so
// nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssm_kernels.h"

namespace ssm {

namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace ssm
