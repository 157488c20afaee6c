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

#include <type_traits>

namespace fp4g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kFmtFp8 = 0;   // OCP E4M3
constexpr int kFmtFp4 = 4;   // E2M1

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous global -> LDS copies (global_load_lds_dwordx4 / _dword): lane i writes
// 16 (or 4) bytes at offset 16*i (4*i) after the wave-uniform LDS address.  The
// builtin is only spelled in the device pass: in the host pass its presence in a
// kernel body suppresses the kernel's launch stub.
__device__ __forceinline__ void lds_copy16(const void* g, lds_void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#else
  (void)g;
  (void)l;
#endif
}
// The same copy with the nontemporal cache policy, for data read exactly once.
__device__ __forceinline__ void lds_copy16_nt(const void* g, lds_void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2);
#else
  (void)g;
  (void)l;
#endif
}
__device__ __forceinline__ void lds_copy4(const void* g, lds_void* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
#else
  (void)g;
  (void)l;
#endif
}

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits only for this wave's LDS operations (lgkmcnt), not
// for its in-flight global->LDS copies: those are waited for explicitly with
// wait_vmcnt, which keeps later ring stages in flight across the barrier.  The
// signal fences stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// fp32 -> bf16 bits with gfx950's v_cvt_pk_bf16_f32: round to nearest even, NaN stays
// NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values -> packed bf16x2 (low half = a), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float v2f_ __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_ __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_{a, b}), v2bf_));
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

// Store four consecutive output elements D[idx .. idx+3] of type OUT; only the first
// `avail` exist when the row ends inside the group.  A whole group goes out as one
// 8-byte (bf16) or 16-byte (fp32) store when its address is aligned for it.
template <bool BF16>
__device__ __forceinline__ void store_out4(void* D, int64_t idx, int avail, float v0, float v1, float v2,
                                           float v3) {
  if constexpr (BF16) {
    uint16_t* p = reinterpret_cast<uint16_t*>(D) + idx;
    const uint32_t w01 = pack_bf16x2(v0, v1), w23 = pack_bf16x2(v2, v3);
    if (avail >= 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      typedef unsigned int v2u __attribute__((ext_vector_type(2)));
      *reinterpret_cast<v2u*>(p) = v2u{w01, w23};
    } else {
      if (avail > 0) p[0] = (uint16_t)w01;
      if (avail > 1) p[1] = (uint16_t)(w01 >> 16);
      if (avail > 2) p[2] = (uint16_t)w23;
      if (avail > 3) p[3] = (uint16_t)(w23 >> 16);
    }
  } else {
    float* p = reinterpret_cast<float*>(D) + idx;
    if (avail >= 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<v4f*>(p) = v4f{v0, v1, v2, v3};
    } else {
      if (avail > 0) p[0] = v0;
      if (avail > 1) p[1] = v1;
      if (avail > 2) p[2] = v2;
      if (avail > 3) p[3] = v3;
    }
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

// Calls f(integral_constant<int, I>) for I = B .. E-1 (each a compile-time constant).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Integer helpers.
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace fp4g
