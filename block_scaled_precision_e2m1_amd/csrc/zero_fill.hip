// D = 0 for a product with an empty K range.  A plain store kernel rather than
// hipMemsetAsync, so a caller may capture the call in a HIP graph.
#include <atomic>

#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

__global__ void __launch_bounds__(256) zero_fill_kernel(uint32_t* __restrict__ p, int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

__global__ void zero_tail_kernel(uint16_t* __restrict__ p) { *p = 0; }

}  // namespace

// The count is cached per device in atomics: host threads may call the library at
// once, and a first query racing another only stores the same value twice.
int64_t device_cus() {
  static std::atomic<int64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int64_t n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int q = 0;
    if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || q <= 0) q = 256;
    n = q;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_zero_fill(void* D, int64_t count, bool bf16_out, hipStream_t s) {
  const int64_t bytes = count * (bf16_out ? 2 : 4);
  const int64_t words = bytes / 4;
  if (words > 0) {
    const int64_t blocks = ceil_div(words, 256) < 4096 ? ceil_div(words, 256) : 4096;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(D), words);
  }
  if (bytes % 4)   // an odd number of bf16 elements leaves one half-word
    hipLaunchKernelGGL(zero_tail_kernel, dim3(1), dim3(1), 0, s,
                       reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(D) + bytes - 2));
  return hipGetLastError();
}

}  // namespace fp4g
