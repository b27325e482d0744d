// Library-owned device scratch for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` stands in for the grouped calls' workspace: the gate/up kernels
// store the number of out-of-range slot ids there.  Every GPU holds its own
// copy of the array for the life of the process; its device address is
// resolved once per device with hipGetSymbolAddress and kept, and only that
// address is handed to kernels and copies (the array's name in host code is a
// host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "q4moe_launch.h"

namespace q4 {

namespace {

constexpr size_t kScratchBytes = 256;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // the current device is `dev`: this resolves that device's copy
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace q4
