// Measured ceilings of the chip, reported by the benchmark beside the datasheet peaks.
//
//   fp4p_mfma_probe: every wave of the grid runs `iters` rounds of 12 independent chains
//     of the scaled FP4 32x32x64 matrix instruction on register operands holding random
//     bits (the GEMM's instruction, with its operand toggling), so the time is that of
//     the matrix pipe alone at the clock the chip holds under it.  Wave 0 of each
//     workgroup records the shader clock counter and the 100 MHz constant counter at its
//     start and end, which give the clock the matrix pipe ran at.
//   fp4p_timestamp: every workgroup writes its XCC id, the shader clock counter and the
//     100 MHz constant counter; two of them around a run of kernels on one stream give
//     the average shader clock of each XCC over that run.
//   fp4p_read_probe: streams `bytes` from device memory with 16-byte non-temporal loads
//     (each byte once, every lane in flight with several loads), the attainable read
//     rate of HBM for a buffer past the 256 MB last-level cache.
// Not part of the library's operations: a separate shared library for the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

constexpr int kChains = 12;   // independent accumulator chains per wave (192 accumulator registers)

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, uint64_t seed, float* sink, uint64_t* clocks) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = i < 4 ? (int)hash32(t * 16u + i + (uint32_t)seed) : 0;
    b[i] = i < 4 ? (int)hash32(t * 16u + 8 + i + (uint32_t)(seed >> 32)) : 0;
  }
  v16f acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) { t0 = __builtin_amdgcn_s_memtime(); r0 = __builtin_amdgcn_s_memrealtime(); }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
  sink[t] = s;
}

__global__ void __launch_bounds__(256) read_probe_kernel(const v4i* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4i v0 = __builtin_nontemporal_load(src + i);
    const v4i v1 = __builtin_nontemporal_load(src + i + stride);
    const v4i v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4i v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= (uint32_t)(v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3]);
    x ^= (uint32_t)(v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3]);
  }
  for (; i < n16; i += stride) {
    const v4i v = __builtin_nontemporal_load(src + i);
    x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// Each workgroup (one per CU) records its XCC (hardware register XCC_ID, 4 bits), the
// shader clock counter and the 100 MHz counter.  The shader clock counters of different
// XCCs are not aligned with one another, so clocks are taken per XCC.
__global__ void timestamp_kernel(uint64_t* out) {
  if (threadIdx.x == 0) {
    const uint64_t t = __builtin_amdgcn_s_memtime(), r = __builtin_amdgcn_s_memrealtime();
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u;   // XCC_ID[3:0]
    out[3 * blockIdx.x + 0] = xcc;
    out[3 * blockIdx.x + 1] = t;
    out[3 * blockIdx.x + 2] = r;
  }
}

}  // namespace

extern "C" {

// out: 3 * grid uint64 of device memory: per workgroup (XCC id, shader clock counter,
// 100 MHz counter).
int fp4p_timestamp(int grid, uint64_t* out, void* stream) {
  if (grid <= 0 || !out) return 1;
  hipLaunchKernelGGL(timestamp_kernel, dim3(grid), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// grid workgroups of 4 waves (256 threads); sink: grid*256 floats, clocks: grid*4 uint64.
int fp4p_mfma_probe(int grid, int iters, uint64_t seed, float* sink, uint64_t* clocks, void* stream) {
  if (grid <= 0 || iters <= 0 || !sink || !clocks) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), iters,
                     seed, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// src: bytes (a multiple of 16, 16-byte aligned) of device memory; sink: grid*256 uint32.
int fp4p_read_probe(int grid, const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (grid <= 0 || !src || !sink || bytes <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
