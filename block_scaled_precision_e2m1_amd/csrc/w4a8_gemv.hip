// W4A8 decode GEMV for gfx950: D[M][N] for 1 <= M <= 16 tokens, the same product as
// the W4A8 GEMM,
//   D[m][n] = sa[m] * sum_g sB[n][g] * sum_{k in g} e4m3(A[m][k]) * int4(B[n][k]),
// K groups of 128 elements.
//
// The Hopper CUTLASS/CuTe DSL post (section "What changes in the W4A8 builder") sizes
// the token tile from 16 so that a decode step with a handful of tokens does not pay
// for a 64-token instruction; with the operands swapped (section "The W4A8 kernel: the
// same four definitions, with the operands swapped") the weights fill the 16-row slot
// of the FP8 16x16x128 instruction and the tokens sit in the other slot, zero past M.
// The product computed is D^T = B * A^T: accumulator lane l holds rows n = 4*(l/16)+t
// of one 16-row weight group and token m = l%16.
//
// gfx950 mapping (K <= 16384, the decode shapes), as in the MXFP4 GEMV:
//   * one workgroup of 8 waves per RG groups of 16 weight rows; wave w owns the ST
//     consecutive K groups starting at w*ST for all of the workgroup's rows, so its
//     token fragments are loaded once and reused for every row group;
//   * lane (r, slot) of a K group holds its 32 consecutive K elements 32*slot..+31 in
//     both operands: 16 bytes of INT4 for weight row r and 32 bytes of FP8 for token
//     r, so every aligned run of 8 instruction elements is 8 consecutive K;
//   * the weights reach LDS through global->LDS copies: plain weights [N][K/2] in
//     whole-line 1 KB copies of RPI rows x ST*64 bytes, their 16-byte units XOR-
//     swizzled by row so the 16-row ds_read_b128 hits distinct bank groups; pre-packed
//     weights (w4a8_prepacked.hip: the 16 x 128 operand of one instruction stored lane
//     by lane) in one 1 KB copy per K group, with their fp32 scales beside them;
//   * every load is issued up front and waited for once: a decode GEMV is one pass
//     over a cold weight stream, and what matters is how many bytes are in flight;
//   * each weight dword becomes two exact FP8 operands, E4M3(v) and -s * 2^-6 scaled
//     by 2^9 in the instruction, for q = v - 8s (v the low 3 bits, s bit 3), so two
//     chained instructions over the same tokens give the group's INT4 product; the
//     group's partial tile is folded into the fp32 accumulator times sB[n][g];
//   * the 8 partial tiles of a row group are summed through LDS (reusing the weight
//     area) in wave order, so results are run-to-run identical, then scaled by sa[m].
// K groups past K (the last segment of a ragged K) read clamped in-bounds addresses and
// are given zero tokens and zero scales; rows past N read row N-1 (plain) or the zero
// padding rows (pre-packed) and are not stored.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int WAVES = 8;
constexpr int kMaxGroups = 128;             // K <= 16384: 8 waves x 16 groups

// E4M3 codes of 0..7 as a v_perm_b32 table: selector k picks byte k of {hi:lo}.
constexpr uint32_t kE4M3Lo = 0x44403800u;   // 0, 1, 2, 3
constexpr uint32_t kE4M3Hi = 0x4E4C4A48u;   // 4, 5, 6, 7
constexpr int kScale2p9 = 0x88888888;       // E8M0 136 = 2^9 in every byte

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __builtin_bit_cast(float, u16 << 16); }

template <int NJ, int RG, bool PACKED, bool BF16>
__global__ void __launch_bounds__(WAVES * 64)
w4a8_gemv_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sa,
                 const uint8_t* __restrict__ Bw, const void* __restrict__ Sw, void* __restrict__ D) {
  constexpr int ST = 4 * NJ;                 // K groups (64 bytes of INT4 per row) per wave
  constexpr int SEG = ST * 64;               // plain: bytes per row per wave
  constexpr int UPR = SEG / 16;              // plain: 16-byte units per row segment
  constexpr int RPI = 64 / UPR;              // plain: rows per 1 KB copy
  constexpr int ROWS = 16 * RG;
  constexpr int NI = PACKED ? RG * ST : ROWS / RPI;        // weight copies per wave
  constexpr int SOFF = RG * ST * 1024;       // pre-packed: fp32 scales after the weights
  constexpr int WBYTES = PACKED ? SOFF + RG * ST * 64 : ROWS * SEG;
  constexpr int RED = WAVES * RG * 64 * 16;
  static_assert(UPR >= 16 && UPR <= 64 && 64 % UPR == 0, "segment shape");
  static_assert(WAVES * WBYTES <= 160 * 1024 && RED <= WAVES * WBYTES, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[WAVES * WBYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int KT = K / 128;
  const int ks0 = wave * ST;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const uint16_t* sB = static_cast<const uint16_t*>(Sw);
  if constexpr (!PACKED) {  // plain operands: problem blockIdx.y of a batch stored back to back
    const int64_t b = blockIdx.y;
    A += b * M * K;
    sa += b * M;
    Bw += b * N * (K / 2);
    sB += b * N * KT;
    D = static_cast<uint8_t*>(D) + b * M * N * (BF16 ? 2 : 4);
  }
  uint8_t* wl = lds + wave * WBYTES;

  // ---- tokens of this wave's segment: lanes r >= M read token 0 (the same lines as
  // lanes r = 0) and are zeroed below, as are groups past K ----
  const int64_t trow = r < M ? r : 0;
  v4i t0[ST], t1[ST];
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const uint8_t* p = A + trow * K + (int64_t)min(ks0 + s, KT - 1) * 128 + slot * 32;
    t0[s] = *reinterpret_cast<const v4i*>(p);
    t1[s] = *reinterpret_cast<const v4i*>(p + 16);
  }

  // ---- weights (and, pre-packed, their scales) into this wave's LDS area ----
  const int G16 = (N + 15) / 16;
  if constexpr (PACKED) {
    const int64_t Np = 16 * (int64_t)G16;
    const float* Sp = static_cast<const float*>(Sw);
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int64_t g16 = min(n0 / 16 + g, (int64_t)G16 - 1);
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const int ks = min(ks0 + s, KT - 1);
        lds_copy16_nt(Bw + (g16 * KT + ks) * 1024 + lane * 16, (lds_void*)(wl + (g * ST + s) * 1024));
      }
      // Sp[ks][16*g16 + row]: lane l copies the scale of row l%16 of group 4c + l/16
#pragma unroll
      for (int c = 0; c < ST / 4; ++c) {
        const int ks = min(ks0 + 4 * c + (lane >> 4), KT - 1);
        lds_copy4(Sp + ks * Np + g16 * 16 + r, (lds_void*)(wl + SOFF + (g * ST + 4 * c) * 64));
      }
    }
  } else {
    const int64_t ld = K / 2;
    const int u = lane % UPR, rr = lane / UPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + rr;
      const int gu = u ^ (row & 15);                      // global unit held by LDS unit u
      const int ks = min(ks0 + (gu >> 2), KT - 1);
      const int64_t grow = min(n0 + row, (int64_t)N - 1);
      lds_copy16_nt(Bw + grow * ld + (int64_t)ks * 64 + (gu & 3) * 16, (lds_void*)(wl + i * 1024));
    }
  }

  // ---- plain bf16 group scales: lane (r, slot) needs rows 4*slot + t of each row
  // group, groups ks0 .. ks0+ST-1, kept as bf16 pairs (group 2j in the low half) ----
  constexpr int SW = PACKED ? 1 : ST / 2;
  uint32_t sr[RG][4][SW];
  if constexpr (!PACKED) {
    // Whole-segment vector loads when the segment lies inside the row and the row
    // pitch and base keep them aligned: 16 bytes (8 groups), or 8 bytes for ST = 4.
    constexpr int VB = ST >= 8 ? 16 : 8;
    const bool vec = ks0 + ST <= KT && (KT * 2) % VB == 0 && (reinterpret_cast<uintptr_t>(sB) & (VB - 1)) == 0;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t* p = sB + min(n0 + 16 * g + 4 * slot + t, (int64_t)N - 1) * KT;
        if (vec) {
          if constexpr (VB == 16) {
#pragma unroll
            for (int c = 0; c < ST / 8; ++c) {
              const v4i x = *reinterpret_cast<const v4i*>(p + ks0 + 8 * c);
              sr[g][t][4 * c] = (uint32_t)x[0]; sr[g][t][4 * c + 1] = (uint32_t)x[1];
              sr[g][t][4 * c + 2] = (uint32_t)x[2]; sr[g][t][4 * c + 3] = (uint32_t)x[3];
            }
          } else {
            typedef unsigned int v2u __attribute__((ext_vector_type(2)));
            const v2u x = *reinterpret_cast<const v2u*>(p + ks0);
            sr[g][t][0] = x[0]; sr[g][t][1] = x[1];
          }
        } else {
#pragma unroll
          for (int j = 0; j < SW; ++j)
            sr[g][t][j] = (uint32_t)p[min(ks0 + 2 * j, KT - 1)] | ((uint32_t)p[min(ks0 + 2 * j + 1, KT - 1)] << 16);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);          // every load of this wave, copies included
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  const bool tok = r < M;
  v4f acc[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
  const int unit = 0x7F7F7F7F;
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const bool ok = ks0 + s < KT;
    const v8i tv = tok && ok ? v8i{t0[s][0], t0[s][1], t0[s][2], t0[s][3], t1[s][0], t1[s][1], t1[s][2], t1[s][3]}
                             : v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      v4i x;
      v4f sc;
      if constexpr (PACKED) {
        x = *reinterpret_cast<const v4i*>(wl + (g * ST + s) * 1024 + lane * 16);
        sc = *reinterpret_cast<const v4f*>(wl + SOFF + (g * ST + s) * 64 + slot * 16);
      } else {
        const int row = 16 * g + r;
        x = *reinterpret_cast<const v4i*>(wl + row * SEG + (((s * 4 + slot) ^ r) * 16));
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[t] = bf16_bits_to_f32((sr[g][t][s / 2] >> (16 * (s & 1))) & 0xFFFFu);
      }
      v8i bv, bs;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // Elements 0..3 and 4..7 of the dword in the low nibbles of the bytes of lo and
        // hi.  Pre-packed weights are stored that way; plain ones (byte j holds elements
        // 2j, 2j+1) take one byte permute each of x and x >> 4.
        const uint32_t xw = (uint32_t)x[w], xs = xw >> 4;
        const uint32_t lo = PACKED ? xw : __builtin_amdgcn_perm(xs, xw, 0x05010400u);
        const uint32_t hi = PACKED ? xs : __builtin_amdgcn_perm(xs, xw, 0x07030602u);
        bv[2 * w] = (int)__builtin_amdgcn_perm(kE4M3Hi, kE4M3Lo, lo & 0x07070707u);
        bv[2 * w + 1] = (int)__builtin_amdgcn_perm(kE4M3Hi, kE4M3Lo, hi & 0x07070707u);
        bs[2 * w] = (int)((lo & 0x08080808u) | 0x80808080u);
        bs[2 * w + 1] = (int)((hi & 0x08080808u) | 0x80808080u);
      }
      v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, tv, v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp8, kFmtFp8,
                                                                  0, unit, 0, unit);
      part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bs, tv, part, kFmtFp8, kFmtFp8, 0, kScale2p9, 0, unit);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[g][t] = __builtin_fmaf(part[t], ok ? sc[t] : 0.0f, acc[g][t]);
    }
  }

  // ---- sum the WAVES partial tiles in wave order, scale by sa[m], store D[m][n] ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);   // [WAVES][RG][64 lanes][4]
#pragma unroll
  for (int g = 0; g < RG; ++g) *reinterpret_cast<v4f*>(red + ((wave * RG + g) * 64 + lane) * 4) = acc[g];
  __syncthreads();
  if (threadIdx.x < RG * 64) {
    const int g = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int m = l & 15;
    v4f v = *reinterpret_cast<const v4f*>(red + (g * 64 + l) * 4);
#pragma unroll
    for (int w2 = 1; w2 < WAVES; ++w2) v += *reinterpret_cast<const v4f*>(red + ((w2 * RG + g) * 64 + l) * 4);
    const int64_t n = n0 + 16 * g + 4 * (l >> 4);
    if (m < M && n < N) {
      const float s = sa[m];
      const int avail = (int)min((int64_t)4, (int64_t)N - n);
      store_out4<BF16>(D, (int64_t)m * N + n, avail, v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    }
  }
}

template <int NJ, int RG, bool PACKED>
hipError_t launch_cfg(const W4A8Args& a, const void* S, hipStream_t s) {
  const int64_t g64 = ceil_div(a.N, 16 * RG);
  if (g64 > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)g64, PACKED ? 1u : (unsigned)a.L), block(WAVES * 64);
  if (a.bf16_out)
    hipLaunchKernelGGL((w4a8_gemv_kernel<NJ, RG, PACKED, true>), grid, block, 0, s, (int)a.M, (int)a.N, (int)a.K,
                       a.A, a.sa, a.B, S, a.D);
  else
    hipLaunchKernelGGL((w4a8_gemv_kernel<NJ, RG, PACKED, false>), grid, block, 0, s, (int)a.M, (int)a.N, (int)a.K,
                       a.A, a.sa, a.B, S, a.D);
  return hipGetLastError();
}

template <bool PACKED>
hipError_t launch_shape(const W4A8Args& a, const void* S, hipStream_t s) {
  const int64_t KT = a.K / 128;
  // Segment of ST = 4*NJ groups per wave, WAVES segments per row: K <= WAVES*ST*128.
  if (KT <= WAVES * 4) return launch_cfg<1, 2, PACKED>(a, S, s);     // K <= 4096: 32 rows per workgroup
  if (KT <= WAVES * 8) return launch_cfg<2, 1, PACKED>(a, S, s);     // K <= 8192
  return launch_cfg<4, 1, PACKED>(a, S, s);                          // K <= 16384
}

}  // namespace

bool w4a8_gemv_fits(int64_t M, int64_t K) { return M >= 1 && M <= 16 && K >= 128 && K / 128 <= kMaxGroups; }

hipError_t launch_w4a8_gemv(const W4A8Args& a, const float* Sp, hipStream_t s) {
  if (!w4a8_gemv_fits(a.M, a.K) || a.K % 128 != 0) return hipErrorInvalidValue;
  return Sp ? launch_shape<true>(a, Sp, s) : launch_shape<false>(a, a.sB, s);
}

}  // namespace fp4g
