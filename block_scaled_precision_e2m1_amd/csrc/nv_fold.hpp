// The exact NVFP4 fold shared by the NVFP4 GEMM and GEMV: E2M1 codes times their E4M3
// block scale, widened to fp16.  Every product e2m1 * e4m3 has at most 6 significant
// bits and lies in [2^-10, 2880], inside fp16's normal range, so the fold is exact:
// the scale s = 2^e * m (1 <= m < 2, 3 fraction bits) is applied in two exact steps,
// v_cvt_scalef32_pk_f16_fp4 (two codes widened and multiplied by the power of two of
// its fp32 scale operand, 2^e) and one v_pk_mul_f16 by (m, m).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4g {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// An E4M3 scale byte as the two factors of the fold: `pow2` (fp32; only its power
// of two is used by the conversion) and `mant` = (m, m) in fp16 with the scale's
// sign.  A NaN code (0x7F / 0xFF) gives mant = NaN, so the block's products are NaN.
__device__ __forceinline__ void e4m3_split(uint32_t b, float* pow2, h2* mant) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  uint32_t m16 = 0x3C00u | ((u >> 13) & 0x3FFu) | ((u >> 16) & 0x8000u);
  if ((b & 0x7Fu) == 0x7Fu) m16 = 0x7E00u;
  *pow2 = s;
  *mant = __builtin_bit_cast(h2, m16 | (m16 << 16));
}

// 4 packed bytes (8 E2M1 codes) times one E4M3 scale -> 8 fp16 in 4 dwords.
__device__ __forceinline__ void fold8(uint32_t w, float pow2, h2 mant, uint32_t* out) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 0) * mant);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 1) * mant);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 2) * mant);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, 3) * mant);
}

}  // namespace fp4g
