// W4A8 mixed-input GEMM for gfx950: FP8 E4M3 activations times signed INT4
// weights with one bf16 scale per weight row per 128-element K group and one
// fp32 scale per activation row:
//   D[m][n] = sa[m] * sum_g sB[n][g] * sum_{k in g} e4m3(A[m][k]) * int4(B[n][k])
// This is the W4A8 kernel of the Hopper CUTLASS/CuTe DSL post (sections "The W4A8
// kernel: the same four definitions, with the operands swapped" -- the K tile of
// 128 elements for the 8-bit MMA type, 64 bytes of INT4 -- and "What changes in
// the W4A8 builder": the narrow operand is converted in registers before the MMA,
// and each stage carries one scale per weight row per K tile).  The per-row
// activation scale is applied in the epilogue.
//
// gfx950 design: INT4 -> FP8 is exact for -8..7, so the weights are converted
// while being staged into LDS (two v_perm_b32 table lookups per 4 nibbles, one
// for 0..7 and one for -8..-1, merged with v_bfi_b32, then re-interleaved into K
// order).  One K step is one 128-element group: two
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales) per 32x32 block compute the
// group's partial sum into fresh registers, which is then folded into the fp32
// accumulator with one FMA by the group scale (exact group partials up to the
// MFMA's internal summation).  The next group's tiles are prefetched into
// registers while the current group's MFMAs run.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int kBK = 128;    // one scale group per step
constexpr int kRow = 128;   // bytes of FP8 per LDS row per step

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// Four INT4 nibbles (one per byte, bits 0..3) -> four E4M3 codes.
__device__ __forceinline__ uint32_t int4x4_to_e4m3(uint32_t v) {
  const uint32_t idx = v & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, idx);  // 0..7
  const uint32_t neg = __builtin_amdgcn_perm(0xB8C0C4C8u, 0xCACCCED0u, idx);  // -8..-1
  const uint32_t mask = ((v >> 3) & 0x01010101u) * 0xFFu;
  return (neg & mask) | (pos & ~mask);
}

// Eight packed INT4 (one dword, low nibble = even k) -> eight E4M3 bytes in k order.
__device__ __forceinline__ void int4x8_to_e4m3(uint32_t x, uint32_t* o0, uint32_t* o1) {
  const uint32_t ev = int4x4_to_e4m3(x & 0x0F0F0F0Fu);          // k = 0, 2, 4, 6
  const uint32_t od = int4x4_to_e4m3((x >> 4) & 0x0F0F0F0Fu);   // k = 1, 3, 5, 7
  *o0 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  *o1 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

template <int BM, int BN, int WM, int WN, bool BF16>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
w4a8_gemm_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sa,
                 const uint8_t* __restrict__ B, const uint16_t* __restrict__ sB, void* __restrict__ D) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int CA = BM * 8 / NT;   // 16-byte FP8 chunks of A per thread per step
  constexpr int CB = BN * 4 / NT;   // 16-byte INT4 chunks of B per thread per step
  constexpr int FI = WM / 32, FJ = WN / 32;
  static_assert(CA >= 1 && CB >= 1 && BM * 8 % NT == 0 && BN * 4 % NT == 0, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t la_[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t lb_[2][BN * kRow];
  __shared__ float ls_[2][BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int hi = lane >> 5, r32 = lane & 31;
  {  // problem blockIdx.y of a batch stored back to back
    const int64_t b = blockIdx.y;
    A += b * M * K;
    sa += b * M;
    B += b * N * (K / 2);
    sB += b * N * (K / 128);
    D = static_cast<uint8_t*>(D) + b * M * N * (BF16 ? 2 : 4);
  }
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (int)(blockIdx.x / tiles_n) * BM, n0 = (int)(blockIdx.x % tiles_n) * BN;
  const int G = K / kBK;
  const int64_t ldb = K / 2;

  const uint8_t* ga[CA];
  int oa[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + i * NT, row = q >> 3, c = q & 7;
    ga[i] = A + (int64_t)min(m0 + row, M - 1) * K + c * 16;
    oa[i] = row * kRow + ((c ^ swz8(row)) << 4);
  }
  const uint8_t* gb[CB];
  int ob0[CB], ob1[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = tid + i * NT, row = q >> 2, c = q & 3;   // 16 packed bytes = 32 k = FP8 chunks 2c, 2c+1
    gb[i] = B + (int64_t)min(n0 + row, N - 1) * ldb + c * 16;
    ob0[i] = row * kRow + (((2 * c) ^ swz8(row)) << 4);
    ob1[i] = row * kRow + (((2 * c + 1) ^ swz8(row)) << 4);
  }
  const bool sload = tid < BN;
  const uint16_t* gs = sB + (int64_t)min(n0 + (sload ? tid : 0), N - 1) * G;

  v4i pa[CA], pb[CB];
  uint16_t ps = 0;
  auto load_global = [&](int g) {
#pragma unroll
    for (int i = 0; i < CA; ++i) pa[i] = *reinterpret_cast<const v4i*>(ga[i] + (int64_t)g * kBK);
#pragma unroll
    for (int i = 0; i < CB; ++i) pb[i] = *reinterpret_cast<const v4i*>(gb[i] + (int64_t)g * 64);
    if (sload) ps = gs[g];
  };
  auto store_lds = [&](int st) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<v4i*>(&la_[st][oa[i]]) = pa[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) int4x8_to_e4m3((uint32_t)pb[i][d], &o[2 * d], &o[2 * d + 1]);
      *reinterpret_cast<v4i*>(&lb_[st][ob0[i]]) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      *reinterpret_cast<v4i*>(&lb_[st][ob1[i]]) = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
    }
    if (sload) ls_[st][tid] = bf16_to_f32(ps);
  };

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v16f{};
  const int unit = 0x7F7F7F7F;

  load_global(0);
  store_lds(0);
  if (G > 1) load_global(1);
  for (int g = 0; g < G; ++g) {
    const int st = g & 1;
    __syncthreads();
    v16f part[FI][FJ];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c0 = 4 * kk + 2 * hi;   // this lane's two 16-byte chunks of the 64-element half
      v8i af[FI], bf[FJ];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int row = wm * WM + i * 32 + r32;
        const v4i x0 = *reinterpret_cast<const v4i*>(&la_[st][row * kRow + ((c0 ^ swz8(row)) << 4)]);
        const v4i x1 = *reinterpret_cast<const v4i*>(&la_[st][row * kRow + (((c0 + 1) ^ swz8(row)) << 4)]);
        af[i] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int row = wn * WN + j * 32 + r32;
        const v4i x0 = *reinterpret_cast<const v4i*>(&lb_[st][row * kRow + ((c0 ^ swz8(row)) << 4)]);
        const v4i x1 = *reinterpret_cast<const v4i*>(&lb_[st][row * kRow + (((c0 + 1) ^ swz8(row)) << 4)]);
        bf[j] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], kk == 0 ? v16f{} : part[i][j], kFmtFp8, kFmtFp8, 0, unit, 0, unit);
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const float s = ls_[st][wn * WN + j * 32 + r32];
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[i][j][t] = __builtin_fmaf(part[i][j][t], s, acc[i][j][t]);
    }
    if (g + 1 < G) {
      store_lds(st ^ 1);
      if (g + 2 < G) load_global(g + 2);
    }
  }

#pragma unroll
  for (int i = 0; i < FI; ++i) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int m = m0 + wm * WM + i * 32 + 8 * (t >> 2) + 4 * hi + (t & 3);
      const float rs = sa[min(m, M - 1)];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int n = n0 + wn * WN + j * 32 + r32;
        if (m < M && n < N) store_out<BF16>(D, (int64_t)m * N + n, acc[i][j][t] * rs);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const W4A8Args& a, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const int64_t tiles = ceil_div(a.N, BN) * ceil_div(a.M, BM);
  if (tiles > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)tiles, (unsigned)a.L);
  if (a.bf16_out)
    hipLaunchKernelGGL((w4a8_gemm_kernel<BM, BN, WM, WN, true>), grid, dim3(NT), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sa, a.B, a.sB, a.D);
  else
    hipLaunchKernelGGL((w4a8_gemm_kernel<BM, BN, WM, WN, false>), grid, dim3(NT), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sa, a.B, a.sB, a.D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a8_gemm(const W4A8Args& a, hipStream_t s) {
  if (w4a8_gemv_fits(a.M, a.K)) return launch_w4a8_gemv(a, nullptr, s);   // decode: 16-token tiles
  // The ring kernel of the pre-packed path also takes plain weights when the bf16 group
  // scales of a row pair up into aligned dwords: K % 256 == 0 (the C ABI already
  // requires sB to be 4-byte aligned; the check keeps the kernel's assumption local).
  if (a.K % 256 == 0 && (reinterpret_cast<uintptr_t>(a.sB) & 3) == 0) return launch_w4a8_ring(a, s);
  return launch_cfg<128, 64, 64, 32>(a, s);
}

}  // namespace fp4g
