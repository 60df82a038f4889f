// Library-owned device scratch for the entry points that allocate nothing.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// one copy of it until the process ends. In host code its name stands for the
// host-side shadow, not a device address, so the device address is looked up
// per device (hipGetSymbolAddress with that device current) and only that
// address is handed to kernels.
#include <mutex>

#include "rf_launch.hpp"

namespace rf {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace rf
