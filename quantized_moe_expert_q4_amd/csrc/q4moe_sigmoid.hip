// The bf16 sigmoid table of the SwiGLU tail (GATE_UP_SOURCE, diff page 52 of
// @mlx-bun/inference 1.0.0, kernels/glm52/streamed-experts.ts): the bf16
// value of 1 / (1 + exp(-gT)) for the 4096 bf16 gates gT it is not 0, 1/2 or
// 1 for (sig_table_bits), built once per device by a small kernel into a
// file-scope device array.  The gate/up kernels copy it into LDS at start.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "q4moe_device.h"
#include "q4moe_launch.h"

namespace q4 {

namespace {

__device__ __attribute__((aligned(16))) uint16_t g_sig_table[kSigTable];

__global__ __launch_bounds__(256) void sig_table_kernel() {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < kSigTable) g_sig_table[i] = sigmoid_bf16(sig_table_bits(i));
}

std::atomic<const uint16_t*> g_table_ptr[64];
std::mutex g_table_mutex;

}  // namespace

hipError_t sigmoid_table(const uint16_t** table) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  const uint16_t* t = g_table_ptr[device].load(std::memory_order_acquire);
  if (t) {
    *table = t;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_table_mutex);
  t = g_table_ptr[device].load(std::memory_order_acquire);
  if (!t) {
    // built on a private stream and waited for once, so that every later
    // call, on any stream of this device, finds it complete
    hipStream_t s;
    if ((e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking)) != hipSuccess) return e;
    hipLaunchKernelGGL(sig_table_kernel, dim3(kSigTable / 256), dim3(256), 0, s);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    const hipError_t e2 = hipStreamDestroy(s);
    if (e == hipSuccess) e = e2;
    void* addr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_sig_table));
    if (e != hipSuccess) return e;
    t = static_cast<const uint16_t*>(addr);
    g_table_ptr[device].store(t, std::memory_order_release);
  }
  *table = t;
  return hipSuccess;
}

}  // namespace q4
