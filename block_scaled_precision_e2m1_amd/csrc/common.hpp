// Device-side helpers shared by the gfx950 kernels of the block-scaled FP4 GEMM.
//
// Register layouts of the CDNA4 scaled MFMA (v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4)
// used by the kernels, as measured on gfx950 with one-hot and random operands:
//   FP4 (format 4): lane l holds 32 consecutive K elements (16 bytes, low nibble
//     first) of row l % R (R = 16 or 32) in K-slot l / R; the E8M0 byte selected
//     by op_sel from that lane's scale register scales exactly those 32 elements.
//   FP8 (format 0): lane l holds 32 bytes of row l % R; A and B elements in the
//     same (lane-slot, byte) position are multiplied together.
//   Accumulator: 16x16 -> lane l, element t holds C[4*(l/16) + t][l % 16];
//                32x32 -> lane l, element t holds C[8*(t/4) + 4*(l/32) + t%4][l % 32],
//   with rows taken from the first operand and columns from the second.
// Only the pairing of equal slots matters for the product, so a kernel may
// assign any K order to the slots as long as both operands and their scales
// agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kFmtFp8 = 0;   // OCP E4M3
constexpr int kFmtFp4 = 4;   // E2M1

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Store one output element of type OUT (float or bf16 bits) to D[idx].
template <bool BF16>
__device__ __forceinline__ void store_out(void* D, int64_t idx, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(D)[idx] = f32_to_bf16_rne(v);
  } else {
    reinterpret_cast<float*>(D)[idx] = v;
  }
}

// 16-byte FP4 fragment (32 E2M1 codes) widened to the 8-dword MFMA operand.
__device__ __forceinline__ v8i widen(v4i x) {
  v8i r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// Scaled FP4 x FP4 MFMA, 32x32 output, K = 64 (two 32-element scale blocks).
template <int OPSEL>
__device__ __forceinline__ v16f mfma_fp4_32x32(v4i a, v4i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a), widen(b), c, kFmtFp4, kFmtFp4,
                                                         OPSEL, sa, OPSEL, sb);
}

// Scaled FP4 x FP4 MFMA, 16x16 output, K = 128 (four 32-element scale blocks).
template <int OPSEL>
__device__ __forceinline__ v4f mfma_fp4_16x16(v4i a, v4i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(a), widen(b), c, kFmtFp4, kFmtFp4,
                                                          OPSEL, sa, OPSEL, sb);
}

// Integer helpers.
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace fp4g
