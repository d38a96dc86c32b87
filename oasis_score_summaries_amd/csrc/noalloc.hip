// The step workspace held in a device array of the library itself, for callers that
// cannot allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Each GPU the library runs on holds its own copy
// of the array from the library's load until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace oasis {

constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kNoAllocMaxDevices = 64;

// In host code `scratch` names a host-side handle, not device memory: it is only ever
// passed to hipGetSymbolAddress; kernels receive the device address looked up there.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kNoAllocMaxDevices];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // Once per device, with that device current: its copy's own address.
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace oasis
