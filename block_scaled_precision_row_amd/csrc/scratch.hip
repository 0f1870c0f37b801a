// Library-owned device scratch for callers that cannot allocate (graph capture, tight serving
// loops, harnesses that forbid hipMalloc): one file-scope device array per GPU, found through
// hipGetSymbolAddress once per device and then passed to the kernels as a plain pointer.
//
// In host code the array's name is only a host-side stand-in for the symbol; its device address
// is what hipGetSymbolAddress returns, and each device holds its own copy of the array at its
// own address. The array lives until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bsq_launch.hpp"

namespace bsq {

namespace {
constexpr int kScratchDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices];  // per device, set once under the mutex
}  // namespace

hipError_t scratch_buffer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bsq
