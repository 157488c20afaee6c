// MXFP4 GEMV for decode: D[M][N] with 1 <= M <= 16 tokens, the same block-scaled
// E2M1 x E8M0 product as the GEMM (section 1 of the cuda-oxide page "TMA
// Pipelines, Tensor Cores, and ctm-rs Interop"; its "Where to Go Next" table
// lists the MXFP4 GEMV as a workload of its own).
//
// With few tokens the weight operand B (N rows) is the stream that matters, so
// the operands are swapped as in the W4A8 kernel of the Hopper CUTLASS/CuTe DSL
// post (section "The W4A8 kernel: the same four definitions, with the operands
// swapped"): 16 weight rows fill the 16-row slot of the MFMA and the tokens sit
// in the other slot, padded with zero codes up to 16.  The product computed is
// D^T = B * A^T; its accumulator lane l holds D^T rows 4*(l/16)+t, column l%16,
// which is stored straight into row-major D.
//
// gfx950 mapping: one workgroup of KSPLIT waves per 16 weight rows; wave w owns
// a contiguous range of 128-element K steps, issues its weight loads (16 bytes
// per lane, the row's 64 bytes per step spread over 4 lanes) eight steps at a
// time so many bytes are in flight, runs one v_mfma_scale_f32_16x16x128_f8f6f4
// per step, and the KSPLIT partial tiles are summed through LDS.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int KSPLIT = 4;
constexpr int UNROLL = 8;

template <bool BF16>
__global__ void __launch_bounds__(KSPLIT * 64)
fp4_gemv_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, void* __restrict__ D) {
  __shared__ float red[KSPLIT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int64_t ld = K / 2, lds_ = K / 32;
  const int KT = K / 128;
  const int ks0 = (int)((int64_t)wave * KT / KSPLIT), ks1 = (int)((int64_t)(wave + 1) * KT / KSPLIT);

  // Weight row of this lane (clamped for the ragged last group) and token column.
  const int wrow = min(n0 + r, N - 1);
  const uint8_t* wp = B + (int64_t)wrow * ld + slot * 16;
  const uint8_t* wsp = sfB + (int64_t)wrow * lds_ + slot;
  const bool tok = r < M;
  const int trow = tok ? r : 0;
  const uint8_t* tp = A + (int64_t)trow * ld + slot * 16;
  const uint8_t* tsp = sfA + (int64_t)trow * lds_ + slot;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  int ks = ks0;
  for (; ks + UNROLL <= ks1; ks += UNROLL) {
    v4i w[UNROLL], t[UNROLL];
    int ws[UNROLL], ts[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + (int64_t)(ks + u) * 64));
      ws[u] = wsp[(ks + u) * 4];
      t[u] = *reinterpret_cast<const v4i*>(tp + (int64_t)(ks + u) * 64);
      ts[u] = tsp[(ks + u) * 4];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const v4i tv = tok ? t[u] : v4i{0, 0, 0, 0};
      acc = mfma_fp4_16x16<0>(w[u], tv, acc, ws[u], tok ? ts[u] : 127);
    }
  }
  for (; ks < ks1; ++ks) {
    const v4i w = *reinterpret_cast<const v4i*>(wp + (int64_t)ks * 64);
    const v4i t = tok ? *reinterpret_cast<const v4i*>(tp + (int64_t)ks * 64) : v4i{0, 0, 0, 0};
    acc = mfma_fp4_16x16<0>(w, t, acc, wsp[ks * 4], tok ? tsp[ks * 4] : 127);
  }

#pragma unroll
  for (int t = 0; t < 4; ++t) red[wave][lane][t] = acc[t];
  __syncthreads();
  if (wave == 0) {
    // lane: token column m = lane % 16, weight rows n0 + 4*(lane/16) + t.
    const int m = r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = red[0][lane][t];
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) v += red[w][lane][t];
      const int n = n0 + 4 * slot + t;
      if (m < M && n < N) store_out<BF16>(D, (int64_t)m * N + n, v);
    }
  }
}

}  // namespace

hipError_t launch_fp4_gemv(const FP4Args& a, hipStream_t s) {
  const int64_t g64 = ceil_div(a.N, 16);
  if (g64 > INT32_MAX) return hipErrorInvalidConfiguration;
  const unsigned groups = (unsigned)g64;
  if (a.bf16_out)
    hipLaunchKernelGGL(fp4_gemv_kernel<true>, dim3(groups), dim3(KSPLIT * 64), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  else
    hipLaunchKernelGGL(fp4_gemv_kernel<false>, dim3(groups), dim3(KSPLIT * 64), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  return hipGetLastError();
}

}  // namespace fp4g
