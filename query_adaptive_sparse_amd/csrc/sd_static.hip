// The library's static device scratch: the workspace of sparse_decode_step_static, the decode step
// for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, one copy per GPU the library runs on, held until the
// process ends. In host code its name is only a host-side stand-in, not a device address: the
// device address is looked up once per device with hipGetSymbolAddress (with that device current)
// and kept, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sd_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[sd::kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace sd {

int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return int(hipErrorInvalidSymbol);
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return 0;
}

}  // namespace sd
