// Fixed device scratch for the decode entry point that allocates nothing
// (pa_decode_noalloc): callers under graph capture or in serving loops that
// may not call hipMalloc get the decode work plan and partition states in a
// file-scope device array instead of a caller-supplied workspace.
//
// Each device that the library runs on holds its own copy of the array, at
// its own address, until the process ends.  Host code never uses the array's
// name as a device address (on the host it is only a stand-in): the address
// is taken once per device with hipGetSymbolAddress, with that device
// current, and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once taken
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
