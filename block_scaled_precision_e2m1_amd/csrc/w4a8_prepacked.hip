// Pre-packed W4A8 weights and the GEMM that consumes them (gfx950).
//
// The W4A8 product is that of w4a8_gemm,
//   D[m][n] = sa[m] * sum_g sB[n][g] * sum_{k in g} e4m3(A[m][k]) * int4(B[n][k]),
// groups of 128 K elements.  The Hopper CUTLASS/CuTe DSL post (section "The W4A8
// kernel: the same four definitions, with the operands swapped") reports that the
// INT4 -> FP8 conversion method decides the kernel's speed, and that the fast
// method needs the weights re-encoded and re-ordered, and the scales re-packed, once
// when they are loaded.  This file is that load-time step and its kernel, designed
// for gfx950:
//
// Re-pack.  Within every run of 8 consecutive K elements the nibbles are re-ordered so that
// byte j holds element j in its low nibble and element j+4 in its high nibble, and
// the 16-row x 128-K operand of one 16x16x128 instruction is stored lane by lane:
//   Bp[g16][kg][lane][16 B], lane = 16*slot + r, row 16*g16 + r,
//   K = 128*kg + 32*slot + 8*w + (j or j+4) in byte 4*w + j;
//   Sp[kg][n] = the group scale as fp32 (exact from bf16), n < 16*ceil(N/16).
// Rows past N are zero with scale 0.
//
// Conversion.  A two's-complement nibble q = v - 8s (v = its low 3 bits, s = bit 3).
// With the order above, eight nibbles in one dword x give two FP8 operands exactly,
// with seven VALU instructions and no select between tables:
//   E4M3(v): one v_perm_b32 table lookup of (x & 0x07070707), and of x >> 4;
//   -s * 2^-6: (x & 0x08080808) | 0x80808080 (byte 0x88 = -2^-6, 0x80 = -0),
//              taken by the MFMA with an E8M0 scale of 2^9, i.e. as -8s;
// and v + (-8s) = q, so two chained FP8 MFMAs over the same activations compute
// the group's exact INT4 product.  (Splitting instead into 8 + v and -8 - 8s, two
// bit-ORs, makes both halves about three times larger than q; the instruction's
// inexact internal summation then came within 6% of the 1e-5 bar.  An offset-binary
// operand u = q + 8, one MFMA plus a shared activation sum, measured no faster and
// reached 0.63 of the bar against 0.39.)
//
// Kernel.  Workgroup tile BM = 64 tokens x 64 weight rows, 4 waves, wave w owning
// weight rows 16w .. 16w+15 and all BM tokens (each weight converted once per
// workgroup).
// A stage is one K group: BM x 128 B of activations (16-byte chunks XOR-swizzled by
// row), 4 x 1 KB of packed weights, 64 fp32 scales, copied HBM -> LDS by
// global_load_lds into a 6-slot ring with counted waits and one barrier per group.
// The barrier of group g certifies stage g+1, whose fragments are read into a second
// register set while group g is converted and multiplied.
// Weights are the first MFMA operand (v_mfma_scale_f32_16x16x128_f8f6f4), so a lane's
// four accumulators are four consecutive n of one token m; a group's product goes to
// fresh registers and is folded into the fp32 accumulator times sB[n][g] while the
// next group's MFMAs run.  The epilogue multiplies by sa[m].
#include <type_traits>

#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int QBN = 64;          // weight rows per tile
constexpr int QSTAGES = 6;

template <int BM>
struct QCfg {
  static constexpr int FI = BM / 16;                // token blocks per wave
  static constexpr int B_OFF = BM * 128;            // packed weights of the stage
  static constexpr int S_OFF = B_OFF + QBN * 64;    // fp32 group scales
  static constexpr int STAGE = S_OFF + 1024;
  static constexpr int IA = BM * 128 / 1024 / 4;    // 1 KB activation copies per wave
  static constexpr int LOADS = IA + 2;              // + one weight copy + the scale copy
  static_assert(IA >= 1 && BM % 32 == 0, "tile");
  static_assert(QSTAGES * STAGE <= 160 * 1024, "LDS budget");
  static_assert(QSTAGES >= 3 && (QSTAGES - 2) * LOADS < 64, "vmcnt range");
};

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// E4M3 codes of 0..7 as a v_perm_b32 table: selector k picks byte k of {hi:lo}.
constexpr uint32_t kE4M3Lo = 0x44403800u;   // 0, 1, 2, 3
constexpr uint32_t kE4M3Hi = 0x4E4C4A48u;   // 4, 5, 6, 7
constexpr int kScale2p9 = 0x88888888;       // E8M0 136 = 2^9 in every byte

__global__ void __launch_bounds__(256)
w4a8_prepack_weights_kernel(int64_t units, int N, int G, int64_t ld, const uint8_t* __restrict__ B,
                            uint8_t* __restrict__ Bp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63);
    const int64_t gk = u >> 6;
    const int kg = (int)(gk % G);
    const int64_t row = 16 * (gk / G) + (l & 15);
    v4i out = v4i{0, 0, 0, 0};
    if (row < N) {
      const v4i in = *reinterpret_cast<const v4i*>(B + row * ld + (int64_t)kg * 64 + (l >> 4) * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // nibble i of the dword is element 8w+i; byte j of the result = (elem j) | (elem j+4) << 4
        const uint32_t x = (uint32_t)in[w];
        uint32_t y = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) y |= (((x >> (4 * j)) & 15u) | (((x >> (4 * j + 16)) & 15u) << 4)) << (8 * j);
        out[w] = (int)y;
      }
    }
    *reinterpret_cast<v4i*>(Bp + u * 16) = out;
  }
}

__global__ void __launch_bounds__(256)
w4a8_prepack_scales_kernel(int64_t units, int N, int G, int64_t Np, const uint16_t* __restrict__ sB,
                           float* __restrict__ Sp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int64_t n = u % Np, kg = u / Np;
    Sp[u] = n < N ? __builtin_bit_cast(float, (uint32_t)sB[n * G + kg] << 16) : 0.0f;
  }
}

// The same Sp from E4M3 group scales: scale (n, kg) is the byte sB8[(n * G + kg) * stride],
// stride 1 for a plain [N][K/128] array or 8 for the Hopper post's Array<float_e4m3_t, 8>
// packing (section "The W4A8 kernel: the same four definitions, with the operands
// swapped": each FP8 scale stored as an array of 8 elements; the first is read).  Every
// E4M3 value is exact in fp32; a NaN code stays NaN.
__global__ void __launch_bounds__(256)
w4a8_prepack_e4m3_scales_kernel(int64_t units, int N, int G, int64_t Np, const uint8_t* __restrict__ sB8,
                                int stride, float* __restrict__ Sp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int64_t n = u % Np, kg = u / Np;
    Sp[u] = n < N ? __builtin_amdgcn_cvt_f32_fp8((int)sB8[(n * G + kg) * stride], 0) : 0.0f;
  }
}

// PACKED: Bw is Bp and Sw is Sp as laid out above.  Otherwise Bw is the plain
// w4a8_gemm weight B [N][K/2] and Sw its bf16 group scales sB [N][K/128] (K % 256 == 0,
// sB 4-byte aligned): a wave copies its 16 rows x 64 bytes of the group with the
// 16-byte units XOR-swizzled by row (conflict-free reads), the conversion first puts
// the nibbles into K order with two byte permutes per 8 weights, and the scale copy fetches
// the aligned dword holding groups g & ~1 and (g & ~1) + 1 of each row.
// SPLIT: the K groups are cut into S slices of GS groups (GS even, the last slice
// shorter); work item = tile * S + slice, and the slice's fp32 partial product (without
// sa) goes to D = P[L][S][M][N] for launch_scaled_reduce.
template <int BM, bool PACKED, bool SPLIT, bool BF16>
__global__ void __launch_bounds__(256, 2)
w4a8p_gemm_kernel(int M, int N, int K, int S, int GS, const uint8_t* __restrict__ A, const float* __restrict__ sa,
                  const uint8_t* __restrict__ Bw, const void* __restrict__ Sw, void* __restrict__ D) {
  using C = QCfg<BM>;
  constexpr int FI = C::FI;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[QSTAGES * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, slot = lane >> 4;
  if constexpr (!PACKED) {  // plain operands: problem blockIdx.y of a batch stored back to back
    const int64_t b = blockIdx.y;
    A += b * M * K;
    sa += b * M;
    Bw += b * N * (K / 2);
    Sw = static_cast<const uint8_t*>(Sw) + b * N * (K / 128) * 2;
    D = static_cast<uint8_t*>(D) + b * (SPLIT ? S : 1) * M * N * (SPLIT ? 4 : (BF16 ? 2 : 4));
  }

  // Tile order: the token tiles of one weight panel are adjacent (they share it in
  // L2); consecutive ids go to the 8 XCDs in turn and are regrouped per XCD.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + QBN - 1) / QBN;
  const int T = tiles_m * tiles_n * (SPLIT ? S : 1);
  int lin = blockIdx.x;
  if ((T & 7) == 0) lin = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int slice = SPLIT ? lin % S : 0;
  if constexpr (SPLIT) lin /= S;
  const int m0 = (lin % tiles_m) * BM, n0 = (lin / tiles_m) * QBN;
  const int GA = K / 128;                          // groups of the whole K (row pitches)
  const int g0 = SPLIT ? slice * GS : 0;           // this item's groups: g0 .. g0 + G - 1
  const int G = SPLIT ? min(GS, GA - g0) : GA;
  if constexpr (SPLIT) D = static_cast<float*>(D) + (int64_t)slice * M * N;
  const int G16 = (N + 15) / 16;
  const int64_t Np = 16 * (int64_t)G16;

  // ---- copy sources ----
  const uint8_t* ga[C::IA];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) {
    const int row = 8 * (wave * C::IA + i) + (lane >> 3), u = lane & 7;
    ga[i] = A + (int64_t)min(m0 + row, M - 1) * K + (int64_t)g0 * 128 + ((u ^ swz8(row)) << 4);
  }
  const uint8_t* gb;
  // The scale copy: each wave copies the scales of its own 16 weight rows into its own
  // 256-byte slot (lanes 0..15; lanes 16..63 repeat those addresses, which the copy
  // fetches once, into the rest of the slot).
  const uint8_t* gs;                               // scale copy source (4 bytes per lane)
  int64_t gstep_b, gstep_s;                        // bytes per K group
  const int srow = 16 * wave + (lane & 15);
  if constexpr (PACKED) {
    gb = Bw + ((int64_t)min(n0 / 16 + wave, G16 - 1) * GA + g0) * 1024 + lane * 16;
    gs = static_cast<const uint8_t*>(Sw) + ((int64_t)g0 * Np + min((int64_t)n0 + srow, Np - 1)) * 4;
    gstep_b = 1024;
    gstep_s = Np * 4;
  } else {
    const int rr = lane >> 2, u = lane & 3;        // LDS unit u of row rr holds global unit u ^ f(rr)
    gb = Bw + (int64_t)min(n0 + 16 * wave + rr, N - 1) * (K / 2) + (int64_t)g0 * 64 + ((u ^ ((rr >> 2) & 3)) << 4);
    gs = static_cast<const uint8_t*>(Sw) + ((int64_t)min(n0 + srow, N - 1) * GA + g0) * 2;   // g0 even
    gstep_b = 64;
    gstep_s = 0;                                   // the group offset is added per copy
  }

  auto issue = [&](int g) {
    const int gc = min(g, G - 1);                  // past the end: re-read the last group
    uint8_t* base = smem + (g % QSTAGES) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) lds_copy16(ga[i] + (int64_t)gc * 128, (lds_void*)(base + (wave * C::IA + i) * 1024));
    lds_copy16(gb + (int64_t)gc * gstep_b, (lds_void*)(base + C::B_OFF + wave * 1024));
    if constexpr (PACKED) lds_copy4(gs + (int64_t)gc * gstep_s, (lds_void*)(base + C::S_OFF + wave * 256));
    else lds_copy4(gs + (int64_t)(gc & ~1) * 2, (lds_void*)(base + C::S_OFF + wave * 256));
  };

  v4f acc[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const int unit = 0x7F7F7F7F;

#pragma unroll
  for (int p = 0; p < QSTAGES - 1; ++p) issue(p);

  v4f part[2][FI];
  v4f sc[2];
  auto fold = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[i][t] = __builtin_fmaf(part[buf][i][t], sc[buf][t], acc[i][t]);
  };

  // One group's LDS fragments: the wave's weight dwords and scales, and all BM tokens.
  // Two register sets: the next group's are read while this group's are converted
  // and multiplied.
  struct Frag { v4i x; v4f s; v8i af[FI]; };
  Frag fr[2];
  auto load = [&](int g, auto set_c) {
    constexpr int SET = decltype(set_c)::value;    // = g & 1
    const uint8_t* base = smem + (g % QSTAGES) * C::STAGE;
    Frag& f = fr[SET];
    // weight operand of this wave's 16 rows, and their scales (n = 16w + 4slot + t)
    if constexpr (PACKED) {
      f.x = *reinterpret_cast<const v4i*>(base + C::B_OFF + wave * 1024 + lane * 16);
      f.s = *reinterpret_cast<const v4f*>(base + C::S_OFF + wave * 256 + 16 * slot);
    } else {
      f.x = *reinterpret_cast<const v4i*>(base + C::B_OFF + wave * 1024 + r * 64 + ((slot ^ ((r >> 2) & 3)) << 4));
      // g is even in set 0 and odd in set 1: the low or high bf16 of each dword
      const v4i d = *reinterpret_cast<const v4i*>(base + C::S_OFF + wave * 256 + 16 * slot);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        f.s[t] = __builtin_bit_cast(float, SET == 0 ? (uint32_t)d[t] << 16 : (uint32_t)d[t] & 0xFFFF0000u);
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row = 16 * i + r;
      const v4i a0 = *reinterpret_cast<const v4i*>(base + row * 128 + (((2 * slot) ^ swz8(row)) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(base + row * 128 + (((2 * slot + 1) ^ swz8(row)) << 4));
      f.af[i] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  };

  // Group g (BUF = g & 1): stage g+1 has landed and stage g's fragments are in set BUF.
  auto group = [&](int g, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    wait_vmcnt<(QSTAGES - 3) * C::LOADS>();
    barrier_lds();
    issue(g + QSTAGES - 1);
    load(g + 1, std::integral_constant<int, BUF ^ 1>{});
    const Frag& f = fr[BUF];
    sc[BUF] = f.s;
    v8i bv, bs;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = (uint32_t)f.x[w], xs = x >> 4;
      // Elements 0..3 and 4..7 in the low nibbles of the bytes of a and b.  Pre-packed
      // weights are already in that order; plain ones (byte j holds elements 2j, 2j+1)
      // take one byte permute each of x and x >> 4.
      const uint32_t a = PACKED ? x : __builtin_amdgcn_perm(xs, x, 0x05010400u);
      const uint32_t b = PACKED ? xs : __builtin_amdgcn_perm(xs, x, 0x07030602u);
      bv[2 * w] = (int)__builtin_amdgcn_perm(kE4M3Hi, kE4M3Lo, a & 0x07070707u);
      bv[2 * w + 1] = (int)__builtin_amdgcn_perm(kE4M3Hi, kE4M3Lo, b & 0x07070707u);
      bs[2 * w] = (int)((a & 0x08080808u) | 0x80808080u);
      bs[2 * w + 1] = (int)((b & 0x08080808u) | 0x80808080u);
    }
    // All E4M3(v) products first, then the sign products that accumulate onto them, so
    // no MFMA waits for the one just issued; the previous group's fold fills the gap.
#pragma unroll
    for (int i = 0; i < FI; ++i)
      part[BUF][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, f.af[i], v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp8,
                                                                      kFmtFp8, 0, unit, 0, unit);
    if (g > 0) fold(BUF ^ 1);
#pragma unroll
    for (int i = 0; i < FI; ++i)
      part[BUF][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bs, f.af[i], part[BUF][i], kFmtFp8, kFmtFp8, 0,
                                                                      kScale2p9, 0, unit);
  };

  // stage 0 landed: its fragments into set 0
  wait_vmcnt<(QSTAGES - 2) * C::LOADS>();
  barrier_lds();
  load(0, std::integral_constant<int, 0>{});
  int g = 0;
  for (; g + 2 <= G; g += 2) {
    group(g, std::integral_constant<int, 0>{});
    group(g + 1, std::integral_constant<int, 1>{});
  }
  if (g < G) {
    group(g, std::integral_constant<int, 0>{});
    fold(0);
  } else {
    fold(1);
  }
  wait_vmcnt<0>();

  // Epilogue: lane (slot, r) of token block i holds m = 16i + r and the four
  // consecutive n = 16w + 4slot + 0..3.
  const int n = n0 + wave * 16 + 4 * slot;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int m = m0 + 16 * i + r;
    if (m < M && n < N) {
      if constexpr (SPLIT) {
        store_out4<false>(D, (int64_t)m * N + n, N - n, acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      } else {
        const float s = sa[m];
        store_out4<BF16>(D, (int64_t)m * N + n, N - n, acc[i][0] * s, acc[i][1] * s, acc[i][2] * s, acc[i][3] * s);
      }
    }
  }
}

// Groups per K slice for `splits` slices of G groups: an even count (the plain path
// reads its bf16 scales as dwords of two groups), at least 2.
int w4a8_slice_groups(int64_t G, int64_t splits) {
  const int64_t gs = (ceil_div(G, splits) + 1) & ~(int64_t)1;
  return (int)(gs < 2 ? 2 : gs);
}

template <int BM, bool PACKED>
hipError_t launch_bm(const W4A8Args& a, const void* S, int64_t splits, float* P, hipStream_t s) {
  const int64_t G = a.K / 128;
  const int GS = w4a8_slice_groups(G, splits);
  const int64_t slices = splits > 1 ? ceil_div(G, GS) : 1;   // every slice non-empty
  if (slices > (splits > 1 ? splits : 1)) return hipErrorInvalidValue;   // P holds `splits` slices
  const int64_t items = ceil_div(a.M, BM) * ceil_div(a.N, QBN) * slices;
  if (items > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)items, PACKED ? 1u : (unsigned)a.L);
  if (slices > 1) {
    hipLaunchKernelGGL((w4a8p_gemm_kernel<BM, PACKED, true, false>), grid, dim3(256), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, (int)slices, GS, a.A, a.sa, a.B, S, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_scaled_reduce(PACKED ? 1 : a.L, a.M, a.N, (int)slices, P, a.sa, 1.0f, 0, a.D, a.bf16_out, s);
  }
  if (a.bf16_out)
    hipLaunchKernelGGL((w4a8p_gemm_kernel<BM, PACKED, false, true>), grid, dim3(256), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, 1, (int)G, a.A, a.sa, a.B, S, a.D);
  else
    hipLaunchKernelGGL((w4a8p_gemm_kernel<BM, PACKED, false, false>), grid, dim3(256), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, 1, (int)G, a.A, a.sa, a.B, S, a.D);
  return hipGetLastError();
}

}  // namespace

void w4a8_prepack_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes) {
  const int64_t G16 = ceil_div(N, 16), G = K / 128;
  *weight_bytes = G16 * G * 1024;
  *scale_bytes = G * 16 * G16 * 4;
}

hipError_t launch_w4a8_prepack(int64_t N, int64_t K, const uint8_t* B, const uint16_t* sB, uint8_t* Bp, float* Sp,
                               hipStream_t s) {
  const int64_t G16 = ceil_div(N, 16), G = K / 128, Np = 16 * G16;
  const int64_t cap = device_cus() * 8;
  const int64_t wu = G16 * G * 64, su = G * Np;
  const unsigned gw = (unsigned)(ceil_div(wu, 256) < cap ? ceil_div(wu, 256) : cap);
  const unsigned gs = (unsigned)(ceil_div(su, 256) < cap ? ceil_div(su, 256) : cap);
  hipLaunchKernelGGL(w4a8_prepack_weights_kernel, dim3(gw), dim3(256), 0, s, wu, (int)N, (int)G, K / 2, B, Bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(w4a8_prepack_scales_kernel, dim3(gs), dim3(256), 0, s, su, (int)N, (int)G, Np, sB, Sp);
  return hipGetLastError();
}

hipError_t launch_w4a8_prepack_scales(int64_t N, int64_t K, const uint16_t* sB, float* Sp, hipStream_t s) {
  const int64_t G16 = ceil_div(N, 16), G = K / 128, Np = 16 * G16;
  const int64_t cap = device_cus() * 8;
  const int64_t su = G * Np;
  const unsigned gs = (unsigned)(ceil_div(su, 256) < cap ? ceil_div(su, 256) : cap);
  hipLaunchKernelGGL(w4a8_prepack_scales_kernel, dim3(gs), dim3(256), 0, s, su, (int)N, (int)G, Np, sB, Sp);
  return hipGetLastError();
}

hipError_t launch_w4a8_prepack_e4m3(int64_t N, int64_t K, const uint8_t* B, const uint8_t* sB8, int stride,
                                    uint8_t* Bp, float* Sp, hipStream_t s) {
  const int64_t G16 = ceil_div(N, 16), G = K / 128, Np = 16 * G16;
  const int64_t cap = device_cus() * 8;
  const int64_t wu = G16 * G * 64, su = G * Np;
  const unsigned gw = (unsigned)(ceil_div(wu, 256) < cap ? ceil_div(wu, 256) : cap);
  const unsigned gs = (unsigned)(ceil_div(su, 256) < cap ? ceil_div(su, 256) : cap);
  hipLaunchKernelGGL(w4a8_prepack_weights_kernel, dim3(gw), dim3(256), 0, s, wu, (int)N, (int)G, K / 2, B, Bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(w4a8_prepack_e4m3_scales_kernel, dim3(gs), dim3(256), 0, s, su, (int)N, (int)G, Np, sB8, stride,
                     Sp);
  return hipGetLastError();
}

// a.B is the packed weight buffer; Sp the packed fp32 scales.
hipError_t launch_w4a8_gemm_prepacked(const W4A8Args& a, const float* Sp, hipStream_t s) {
  return launch_w4a8_gemm_split(a, Sp, 1, nullptr, s);
}

// Plain weights and bf16 scales (K % 256 == 0, sB 4-byte aligned).
hipError_t launch_w4a8_ring(const W4A8Args& a, hipStream_t s) { return launch_bm<64, false>(a, a.sB, 1, nullptr, s); }

int64_t w4a8_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, bool packed, int64_t requested, int64_t cap) {
  const int64_t G = K / 128;
  // Only the ring kernel splits: not the decode kernel (M <= 32 fills the chip by rows)
  // and not the plain-weight kernel for K % 256 != 0.
  if (L * M * N == 0 || w4a8_gemv_fits(M, K) || (!packed && K % 256 != 0) || G < 4) return 1;
  int64_t smax = G / 2 < kMaxSplits ? G / 2 : kMaxSplits;
  if (cap < smax) smax = cap;
  if (smax < 2) return 1;
  auto slices = [&](int64_t S) { return ceil_div(G, w4a8_slice_groups(G, S)); };
  if (requested > 0) return slices(requested < smax ? requested : smax);
  // Automatic choice: a 64 x 64 item is a chain of K groups at about 0.45 us each plus
  // about 3.5 us of fixed cost, two items share a CU; the partial products cost a write
  // and a read of L*M*N fp32 per slice at about 4 TB/s.  The cheapest S wins; a slice
  // keeps at least 4 groups.
  const int64_t cus = device_cus();
  const int64_t items = (packed ? 1 : L) * ceil_div(M, 64) * ceil_div(N, 64);
  int64_t best = 1;
  double best_t = 0;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t sl = slices(S);
    const int64_t gs = S == 1 ? G : w4a8_slice_groups(G, S);
    if (S > 1 && gs < 4) break;
    const double rounds = (double)ceil_div(items * sl, 2 * cus);
    double t = rounds * ((double)gs * 0.45 + 3.5);
    if (sl > 1) t += (double)(L * M * N) * 4.0 * (double)(2 * sl) / 4.0e6;
    if (S == 1 || t < best_t) { best = sl; best_t = t; }
  }
  return best;
}

hipError_t launch_w4a8_gemm_split(const W4A8Args& a, const float* Sp, int64_t splits, float* P, hipStream_t s) {
  if (w4a8_gemv_fits(a.M, a.K)) return launch_w4a8_gemv(a, Sp, s);       // decode: 16-token tiles
  if (splits > 1 && !P) return hipErrorInvalidValue;
  // 64-token tiles: two workgroups share a CU (79 KB of LDS, at most 256 registers).
  if (Sp) return launch_bm<64, true>(a, Sp, splits, P, s);
  return launch_bm<64, false>(a, a.sB, splits, P, s);
}

}  // namespace fp4g
