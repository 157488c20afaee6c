// Library-held scratch memory for callers that cannot allocate device memory (code
// under graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// split-K partial sums of mx_fp4_gemm_batched_noalloc live in one file-scope device
// array instead of a caller-supplied workspace.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes) until
// the process ends.  In host code the array's name is only a stand-in for the symbol,
// not a device address: its address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current and cached here, and only that address is
// ever handed to kernels.  Every call on one GPU shares that GPU's array, so calls
// that overlap in time on one GPU (two streams, or two host threads) race on it.
#include <mutex>

#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
float* scratch_addr[kMaxDevices];   // per device; nullptr until first looked up

}  // namespace

hipError_t scratch_pointer(float** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_addr[dev] = static_cast<float*>(p);
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace fp4g
