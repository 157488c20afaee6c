// The second pass of the K-split W4A8 and NVFP4 GEMMs: the S partial products
// P[b][s][m][n] (fp32, one per slice of the K groups) summed in slice order and scaled
// as the unsplit kernels' epilogues scale their accumulators,
//   D[b][m][n] = ldexp((sum_s P[b][s][m][n]) * rs[b][m] * gm, ge),
// rs the W4A8 per-token scales (absent for NVFP4: 1) and gm * 2^ge the NVFP4 global
// scale pair (1 for W4A8).  One pass over the partials: four consecutive n per lane when
// N % 4 == 0.  Plain loads: the partials were written just before and may still sit in
// the caches (nontemporal loads measured about 1% slower).
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

template <bool BF16, bool VEC>
__global__ void __launch_bounds__(256)
scaled_reduce_kernel(int64_t M, int64_t N, int L, int S, const float* __restrict__ P,
                     const float* __restrict__ rs, float gm, int ge, void* __restrict__ D) {
  constexpr int W = VEC ? 4 : 1;
  const int64_t MN = M * N, per = MN / W, total = per * L;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (int64_t)gridDim.x * 256) {
    const int64_t b = u / per, i = (u - b * per) * W;
    const float* p = P + b * S * MN + i;
    const float sc = (rs ? rs[b * M + i / N] : 1.0f) * gm;
    if constexpr (VEC) {
      v4f acc = *reinterpret_cast<const v4f*>(p);
      for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const v4f*>(p + s * MN);
      store_out4<BF16>(D, b * MN + i, 4, __builtin_ldexpf(acc[0] * sc, ge), __builtin_ldexpf(acc[1] * sc, ge),
                       __builtin_ldexpf(acc[2] * sc, ge), __builtin_ldexpf(acc[3] * sc, ge));
    } else {
      float acc = p[0];
      for (int s = 1; s < S; ++s) acc += p[s * MN];
      store_out<BF16>(D, b * MN + i, __builtin_ldexpf(acc * sc, ge));
    }
  }
}

}  // namespace

hipError_t launch_scaled_reduce(int64_t L, int64_t M, int64_t N, int S, const float* P, const float* rs, float gm,
                                int ge, void* D, bool bf16_out, hipStream_t s) {
  const bool vec = N % 4 == 0;   // four n of one row per lane, so one row scale
  const int64_t units = L * M * (vec ? N / 4 : N);
  const int64_t cap = device_cus() * 8;
  const unsigned grid = (unsigned)(ceil_div(units, 256) < cap ? ceil_div(units, 256) : cap);
  if (grid == 0) return hipSuccess;
  if (bf16_out) {
    if (vec) hipLaunchKernelGGL((scaled_reduce_kernel<true, true>), dim3(grid), dim3(256), 0, s, M, N, (int)L, S, P, rs, gm, ge, D);
    else hipLaunchKernelGGL((scaled_reduce_kernel<true, false>), dim3(grid), dim3(256), 0, s, M, N, (int)L, S, P, rs, gm, ge, D);
  } else {
    if (vec) hipLaunchKernelGGL((scaled_reduce_kernel<false, true>), dim3(grid), dim3(256), 0, s, M, N, (int)L, S, P, rs, gm, ge, D);
    else hipLaunchKernelGGL((scaled_reduce_kernel<false, false>), dim3(grid), dim3(256), 0, s, M, N, (int)L, S, P, rs, gm, ge, D);
  }
  return hipGetLastError();
}

}  // namespace fp4g
