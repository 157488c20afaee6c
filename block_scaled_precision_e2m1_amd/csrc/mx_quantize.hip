// MX quantizer for gfx950: fp32 or bf16 X[rows][K] -> E2M1 codes [rows][K/2] and
// E8M0 block scales [rows][K/32], the step that turns activations into the MXFP4
// operand of the GEMM and the decode GEMV (the issue page's "Impact" section puts
// FP4 GEMMs in inference; the cute-rs page's "Where to Go Next" table lists the
// MXFP4 GEMV).  The rounding rule is the max-abs rule, per 32-element block:
//   e = clamp(floor(log2 amax) - 2 + 127, 0, 254)   (127 for an all-zero block),
//   code = nearest E2M1 value of x * 2^(127-e), ties to the even mantissa bit,
//          saturating at 6; a zero result is +0;
// a block holding an infinity or NaN gets scale 0xFF and zero codes.
//
// HBM-bound: X is read once, the codes and scales written once.  8 lanes share a
// block (4 elements each), so one wave-wide load is 1 KB (fp32) or 512 B (bf16) of
// consecutive blocks and one 2-byte store per lane writes 128 contiguous code
// bytes.  The block maximum and the non-finite flag are reduced over the 8 lanes
// with lane permutations (no LDS storage).  floor(log2 amax) comes from the
// fp32 exponent field, and the scaling and rounding of two elements are one
// hardware conversion (v_cvt_scalef32_pk_fp4_f32) whose results were checked
// against the rule on a sweep of values, ties and saturation included, and are
// checked bit for bit against the oracle by the tests.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int kUnroll = 8;   // blocks-of-8 per wave per iteration, for loads in flight

// Maximum over the 8-lane group (lanes 8g .. 8g+7) of unsigned integers: a butterfly
// of two DPP quad permutations (partners 1 and 2 apart) and one ds_swizzle that
// exchanges the two quads of the group (partner 4 apart).
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v = v > t ? v : t;
  // swap the two quads of each 8-lane group: lane i <- lane i ^ 4
  t = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);               // xor mask 4 within 32
  v = v > t ? v : t;
  return v;
}

template <bool BF16_IN>
__global__ void __launch_bounds__(256)
mx_quantize_kernel(int64_t nblocks, const void* __restrict__ X, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;                 // position of this lane's 4 elements in the block
  const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  // block handled by this lane in unit u of an iteration: 8 blocks per wave-unit
  for (int64_t base = wave_id * 8 * kUnroll; base < nblocks; base += nwaves * 8 * kUnroll) {
    uint32_t bits[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = min(base + u * 8 + (lane >> 3), nblocks - 1);   // clamped: in bounds
      if constexpr (BF16_IN) {
        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
        const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(static_cast<const uint16_t*>(X) + blk * 32 + sub * 4));
        bits[u][0] = w[0] << 16;
        bits[u][1] = w[0] & 0xFFFF0000u;
        bits[u][2] = w[1] << 16;
        bits[u][3] = w[1] & 0xFFFF0000u;
      } else {
        const v4i w = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const float*>(X) + blk * 32 + sub * 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) bits[u][i] = (uint32_t)w[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = base + u * 8 + (lane >> 3);
      // |x| as ordered integers; any exponent field of all ones marks the block non-finite
      uint32_t amax = 0, bad = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = bits[u][i] & 0x7FFFFFFFu;
        bad |= (a >= 0x7F800000u) ? 1u : 0u;
        amax = a > amax ? a : amax;
      }
      amax = group8_max(amax);
      bad = group8_max(bad);
      const int E = (int)(amax >> 23);                  // biased exponent of the block maximum
      const int e = amax == 0 ? 127 : (E - 2 > 0 ? E - 2 : 0);
      // v_cvt_scalef32_pk_fp4_f32 divides two values by the power of two of its scale
      // operand (here 2^(e-127), whose exponent field is e) and rounds each to the
      // nearest E2M1 value, ties to the even code, saturating at 6: the rule above.  It
      // writes -0 (code 8) for a negative value that rounds to zero; the rule's zero
      // is +0, so the sign bit of every zero magnitude is cleared.
      const float scale = __builtin_bit_cast(float, (uint32_t)e << 23);
      uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __builtin_bit_cast(float, bits[u][0]),
                                                                __builtin_bit_cast(float, bits[u][1]), scale, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, __builtin_bit_cast(float, bits[u][2]),
                                                        __builtin_bit_cast(float, bits[u][3]), scale, 1);
      const uint32_t nonzero = ((packed & 0x7777u) + 0x7777u) & 0x8888u;   // bit 3 of a nibble: magnitude != 0
      packed &= nonzero | 0x7777u;
      if (bad) packed = 0;
      if (blk < nblocks) {
        *reinterpret_cast<uint16_t*>(codes + blk * 16 + sub * 2) = (uint16_t)packed;
        if (sub == 0) scales[blk] = bad ? (uint8_t)0xFF : (uint8_t)e;
      }
    }
  }
}

// ---- NV quantizer ------------------------------------------------------------------------
// fp32 or bf16 X[rows][K] and an fp32 global scale g -> E2M1 codes [rows][K/2] and E4M3
// block scales [rows][K/16], the NVFP4 operand of nv_fp4_gemm (the issue page's "Scale
// Factor Granularity": sf_vec_size 16 with Float8E4M3FN scales).  The rule, per
// 16-element block, on exact real quotients:
//   s = the E4M3 code nearest to amax / (6 g), ties to the even code, past 448
//   saturating to 448;  each element is the E2M1 value nearest to x / (e4m3(s) g), ties
//   to the even code, saturating at 6, zero +0;  a scale that decodes to 0 gives zero
//   codes;  a block holding an infinity or NaN gets scale 0x7F (NaN) and zero codes.
// 4 lanes share a block (4 elements each): one wave-wide load is still 1 KB of
// consecutive blocks.
//
// Fast path in fp32, exact decisions where fp32 could decide wrongly:
//  * Scale: sv = amax / fl(6 g) is within 2 ulps of the exact quotient.  Every E4M3
//    rounding boundary has an fp32 mantissa whose low 19 bits are zero, so an sv more
//    than 64 ulps from such a value decides like the exact quotient.  Otherwise (and
//    when 6 g overflows fp32) the code comes from the fp64 quotient, which decides
//    exactly: 6 g is exact in fp64, and a boundary times 6 g has at most 31 significant
//    bits, so amax differs from it by zero or by at least 2^-32 of its size, far more
//    than the fp64 quotient's rounding.
//  * Elements: y = x * inv with inv = fl(1 / fl(e4m3(s) g)) from an LDS table (127
//    values per call) is within 3 fp32 roundings of the exact quotient, so the exact
//    quotient lies between y (1 - 2^-20) and y (1 + 2^-20).  Rounding to E2M1 is
//    monotone: when both ends give the same codes (one hardware conversion per pair),
//    so does the exact quotient.  When they differ, when e4m3(s) g is not a normal fp32
//    (the table holds -1 there), or when the scale saturated (|y| may then overflow),
//    the lane's four codes come from fp64 quotients x / (e4m3(s) g), exact for the same
//    reason as the scale's (a boundary times the divisor has at most 31 bits); where
//    only the two ends differ, one fused multiply-add per element settles it (below).

// Maximum over the 4-lane quad of unsigned integers.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return v > t ? v : t;
}

// The E4M3FN code nearest to sv >= 0 (+inf allowed), ties to the even code, values past
// 448 saturating to 448 (code 0x7E).  Below 2^-6 the codes are the multiples of 2^-9
// (code 8 = 2^-6 continues into the normal range); above, the fp32 mantissa is rounded
// to 3 bits, ties to even, a carry moving into the exponent.
__device__ __forceinline__ uint32_t e4m3_nearest(float sv) {
  const uint32_t u = __builtin_bit_cast(uint32_t, sv);
  if (u >= 0x43E00000u) return 0x7Eu;                               // sv >= 448
  if (u < 0x3C800000u) return (uint32_t)__builtin_rintf(sv * 512.0f);   // sv < 2^-6: 0 .. 8
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u); // biased exponent E - 127 + 7
  return code > 0x7Eu ? 0x7Eu : code;
}

// The same rounding of the fp64 quotient amax / (6 g): exact (see above).
__device__ __noinline__ uint32_t e4m3_nearest_exact(float amax, float g) {
  const double q = (double)amax / (6.0 * (double)g);
  if (q >= 448.0) return 0x7Eu;
  if (q < 0x1p-6) return (uint32_t)__builtin_rint(q * 512.0);          // 0 .. 8, ties to even
  const uint64_t u = __builtin_bit_cast(uint64_t, q);
  const uint64_t r = u + 0xFFFFFFFFFFFFull + ((u >> 49) & 1u);        // 3 of 52 mantissa bits kept
  const uint32_t code = (uint32_t)((((r >> 52) - 1016u) << 3) | ((r >> 49) & 7u));   // E - 1023 + 7
  return code > 0x7Eu ? 0x7Eu : code;
}

// The E2M1 code nearest to the fp64 quotient x / d (d = e4m3(s) g exactly), ties to the
// even code, saturating at 6, zero +0: the count of rounding boundaries strictly below
// |q|, moved up by one on a tie whose lower neighbour is odd.
__device__ __noinline__ uint32_t e2m1_nearest_exact(float x, double d) {
  const double q = (double)x / d;
  const double a = __builtin_fabs(q);
  uint32_t c = (uint32_t)(a > 0.25) + (uint32_t)(a > 0.75) + (uint32_t)(a > 1.25) + (uint32_t)(a > 1.75) +
               (uint32_t)(a > 2.5) + (uint32_t)(a > 3.5) + (uint32_t)(a > 5.0);
  const double bound = c == 0 ? 0.25 : c == 1 ? 0.75 : c == 2 ? 1.25 : c == 3 ? 1.75 : c == 4 ? 2.5
                     : c == 5 ? 3.5 : 5.0;
  if (c < 7 && a == bound && (c & 1u)) c += 1;
  if (c != 0 && q < 0.0) c |= 8u;
  return c;
}

template <bool BF16_IN>
__global__ void __launch_bounds__(256)
nv_quantize_kernel(int64_t nblocks, const void* __restrict__ X, float g, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3;                 // position of this lane's 4 elements in the block
  const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const float six_g = 6.0f * g;
  const bool six_g_finite = six_g <= 3.40282347e38f;
  // 1 / (e4m3(s) g) for the 127 finite codes, -1 where e4m3(s) g is not a normal fp32
  // (s = 0 included); the workgroup computes them once into LDS.
  __shared__ float inv_tab[128];
  if (threadIdx.x < 128) {
    const float d = __builtin_amdgcn_cvt_f32_fp8((int)threadIdx.x, 0) * g;
    inv_tab[threadIdx.x] = (d >= 1.17549435e-38f && d <= 3.40282347e38f) ? 1.0f / d : -1.0f;
  }
  __syncthreads();
  // 16 blocks per wave-unit
  for (int64_t base = wave_id * 16 * kUnroll; base < nblocks; base += nwaves * 16 * kUnroll) {
    uint32_t bits[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = min(base + u * 16 + (lane >> 2), nblocks - 1);   // clamped: in bounds
      if constexpr (BF16_IN) {
        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
        const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(static_cast<const uint16_t*>(X) + blk * 16 + sub * 4));
        bits[u][0] = w[0] << 16;
        bits[u][1] = w[0] & 0xFFFF0000u;
        bits[u][2] = w[1] << 16;
        bits[u][3] = w[1] & 0xFFFF0000u;
      } else {
        const v4i w = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const float*>(X) + blk * 16 + sub * 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) bits[u][i] = (uint32_t)w[i];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t blk = base + u * 16 + (lane >> 2);
      uint32_t amax = 0, bad = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = bits[u][i] & 0x7FFFFFFFu;
        bad |= (a >= 0x7F800000u) ? 1u : 0u;
        amax = a > amax ? a : amax;
      }
      amax = quad_max(amax);
      bad = quad_max(bad);
      const float amax_f = __builtin_bit_cast(float, amax);
      const float sv = amax_f / six_g;
      uint32_t s = e4m3_nearest(sv);
      const uint32_t usv = __builtin_bit_cast(uint32_t, sv);
      if (!bad && amax != 0 && (!six_g_finite || ((usv + 0x40u) & 0x7FFFFu) <= 0x80u))
        s = e4m3_nearest_exact(amax_f, g);
      const float inv = inv_tab[s];
      const float inv_lo = inv * (1.0f - 0x1p-20f), inv_hi = inv * (1.0f + 0x1p-20f);
      float ylo[4], yhi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ylo[i] = __builtin_bit_cast(float, bits[u][i]) * inv_lo;
        yhi[i] = __builtin_bit_cast(float, bits[u][i]) * inv_hi;
      }
      uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ylo[0], ylo[1], 1.0f, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, ylo[2], ylo[3], 1.0f, 1);
      uint32_t packed_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, yhi[0], yhi[1], 1.0f, 0);
      packed_hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed_hi, yhi[2], yhi[3], 1.0f, 1);
      if (!bad && s != 0 && ((packed ^ packed_hi) & 0xFFFFu || inv < 0.0f || s == 0x7Eu)) {
        const float se = __builtin_amdgcn_cvt_f32_fp8((int)s, 0);
        bool tiny = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t a = bits[u][i] & 0x7FFFFFFFu;
          tiny |= a != 0 && a < 0x0D800000u;             // 0 < |x| < 2^-100
        }
        if (inv < 0.0f || s == 0x7Eu || tiny) {
          const double d = (double)se * (double)g;
          packed = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            packed |= e2m1_nearest_exact(__builtin_bit_cast(float, bits[u][i]), d) << (4 * i);
        } else {
          // The two ends of the bracket give adjacent magnitudes k and k+1 (the bracket is far
          // narrower than the spacing of the E2M1 values), so the exact quotient is decided
          // by the boundary between them, b_k: |x| against b_k * e4m3(s) * g.  b_k * e4m3(s)
          // has at most 7 significant bits (exact in fp32), and one fused multiply-add gives
          // the sign of b_k e4m3(s) g - |x| exactly (|x| >= 2^-100 keeps a nonzero difference
          // above the fp32 underflow); zero is a tie, settled to the even magnitude.
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t kl = (packed >> (4 * i)) & 7u, kh = (packed_hi >> (4 * i)) & 7u;
            if (kl != kh) {
              const float b = kl == 0 ? 0.25f : kl == 1 ? 0.75f : kl == 2 ? 1.25f : kl == 3 ? 1.75f
                            : kl == 4 ? 2.5f : kl == 5 ? 3.5f : 5.0f;
              const float ax = __builtin_bit_cast(float, bits[u][i] & 0x7FFFFFFFu);
              const float r = __builtin_fmaf(b * se, g, -ax);
              const uint32_t k = r > 0.0f ? kl : r < 0.0f ? kh : ((kl & 1u) ? kh : kl);
              packed = (packed & ~(7u << (4 * i))) | (k << (4 * i));
            }
          }
        }
      }
      const uint32_t nonzero = ((packed & 0x7777u) + 0x7777u) & 0x8888u;   // bit 3 of a nibble: magnitude != 0
      packed &= nonzero | 0x7777u;
      if (bad || s == 0) packed = 0;
      if (blk < nblocks) {
        *reinterpret_cast<uint16_t*>(codes + blk * 8 + sub * 2) = (uint16_t)packed;
        if (sub == 0) scales[blk] = bad ? (uint8_t)0x7F : (uint8_t)s;
      }
    }
  }
}

}  // namespace

hipError_t launch_nv_quantize(int64_t rows, int64_t K, const void* X, bool bf16_in, float g, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (K / 16);
  const int64_t units = ceil_div(nblocks, 16 * kUnroll);         // wave-iterations of work
  const int64_t wgs = ceil_div(units, 4);                          // 4 waves per workgroup
  const unsigned grid = (unsigned)(wgs < device_cus() * 8 ? wgs : device_cus() * 8);
  if (bf16_in)
    hipLaunchKernelGGL(nv_quantize_kernel<true>, dim3(grid), dim3(256), 0, s, nblocks, X, g, codes, scales);
  else
    hipLaunchKernelGGL(nv_quantize_kernel<false>, dim3(grid), dim3(256), 0, s, nblocks, X, g, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(int64_t rows, int64_t K, const void* X, bool bf16_in, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (K / 32);
  const int64_t units = ceil_div(nblocks, 8 * kUnroll);          // wave-iterations of work
  const int64_t wgs = ceil_div(units, 4);                          // 4 waves per workgroup
  const unsigned grid = (unsigned)(wgs < device_cus() * 8 ? wgs : device_cus() * 8);
  if (bf16_in)
    hipLaunchKernelGGL(mx_quantize_kernel<true>, dim3(grid), dim3(256), 0, s, nblocks, X, codes, scales);
  else
    hipLaunchKernelGGL(mx_quantize_kernel<false>, dim3(grid), dim3(256), 0, s, nblocks, X, codes, scales);
  return hipGetLastError();
}

}  // namespace fp4g
