// Library-owned device scratch for the allocation-free chunkwise entry point.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from module load until the process ends.
// In host code the array's name is only a host-side stand-in, never a device
// address, so the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; every later use
// goes through that pointer. Calls that use the scratch on one GPU share it:
// they must not overlap in time (the same stream, or streams ordered by the
// caller), and the contents left by a call are not cleared by the next one
// unless the path needs zeros.
#include <hip/hip_runtime.h>

#include <atomic>

#include "kernels.h"

namespace ret {

namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_pointer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace ret
