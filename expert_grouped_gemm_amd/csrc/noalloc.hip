// Library-owned scratch memory for the allocation-free dispatch entry point
// (moe_dispatch_noalloc): a file-scope device array, one copy per GPU, that
// lives until the process ends.
//
// Host code never passes the array's name to a kernel: on the host that name
// is a stand-in, not a device address. The device address is looked up once
// per device, with that device current, by hipGetSymbolAddress, and kept per
// device; every use goes through it.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;  // 8 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// The current device's copy of the scratch array (its address resolved on
// the first call on that device).
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
