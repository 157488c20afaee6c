// MXFP4 GEMV for decode: D[M][N] with 1 <= M <= 32 tokens, the same block-scaled
// E2M1 x E8M0 product as the GEMM (section 1 of the cuda-oxide page "TMA
// Pipelines, Tensor Cores, and ctm-rs Interop"; its "Where to Go Next" table
// lists the MXFP4 GEMV as a workload of its own).
//
// With few tokens the weight operand B (N rows) is the stream that matters, so
// the operands are swapped as in the W4A8 kernel of the Hopper CUTLASS/CuTe DSL
// post (section "The W4A8 kernel: the same four definitions, with the operands
// swapped"): 16 weight rows fill the 16-row slot of the MFMA and the tokens sit
// in the other slot, zero past M.  The product computed is D^T = B * A^T; its
// accumulator lane l holds D^T rows 4*(l/16)+t, column l%16 of a 16-token tile.  With 17
// to 32 tokens (K <= 16384) a second token tile multiplies the same weight fragments.
//
// gfx950 mapping (K <= 16384, the decode shapes):
//   * one workgroup of NWV waves (8; 4 at 7168 < K <= 8192) per RG groups of 16 weight
//     rows; wave w owns the K segment of ST = 4*NJ consecutive 128-element steps
//     starting at w*ST, for all of the workgroup's rows, so its token fragments are
//     loaded once and reused for every row group;
//   * the weights reach LDS through global->LDS copies (global_load_lds_dwordx4)
//     that read whole 128-byte lines: each 1 KB copy covers RPI rows x ST*64 bytes.
//     A row's 16-byte units are XOR-swizzled by the row index (the copy lane picks
//     the global unit, the LDS slot stays linear), so the MFMA-layout
//     ds_read_b128 of 16 rows at one K position hits 16 distinct bank groups;
//   * every load is issued up front (tokens first, then the weight copies, then
//     the scale words) and waited for once: a decode GEMV is one pass over a
//     cold weight stream, and what matters is how many bytes are in flight;
//   * the 8 partial 16-row tiles of a row group are summed through LDS (reusing
//     the weight area) in a fixed order, so results are run-to-run identical.
// Steps past K (the last segment of a ragged K) read clamped in-bounds addresses
// and are given zero tokens and unit scales; rows past N read row N-1 and are
// not stored.  Longer K uses the streaming kernel at the end of this file.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int WAVES = 8;

// NWV waves per workgroup.  HALF (M <= 8, one token tile): lanes 8..15 fetch the next step
// of tokens 0..7.  It is a template parameter, not a test of M in the kernel: with both
// forms in one kernel the compiler merges their token registers where the branches join,
// and the moves it puts there wait for the token loads before a single weight copy has
// been issued.
template <int NJ, int RG, int TT, bool HALF, bool COOP, bool BF16, int NWV>
__global__ void __launch_bounds__(NWV * 64)
fp4_gemv_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, void* __restrict__ D) {
  constexpr int ST = 4 * NJ;             // steps (128 K elements, 64 bytes) per wave
  constexpr int SEG = ST * 64;           // bytes per row per wave
  constexpr int UPR = SEG / 16;          // 16-byte units per row segment
  constexpr int RPI = 64 / UPR;          // rows per 1 KB copy
  constexpr int ROWS = 16 * RG;
  constexpr int NI = ROWS / RPI;         // copies per wave
  constexpr int WBYTES = ROWS * SEG;     // LDS bytes per wave
  static_assert(UPR >= 16 && UPR <= 64 && 64 % UPR == 0, "segment shape");
  static_assert(NWV * WBYTES <= 160 * 1024, "LDS budget");
  static_assert(NWV * RG * TT * 64 * 4 * 4 <= NWV * WBYTES, "reduction fits in the weight area");
  static_assert(TT == 1 || TT == 2, "token tiles");
  static_assert(!HALF || TT == 1, "the half-row token fetch is for one tile");
  constexpr int SCL = COOP ? ROWS * ST * NWV * 4 : 16;   // the workgroup's scale rows (K / 32 bytes each)
  static_assert(NWV * WBYTES + SCL <= 160 * 1024, "LDS budget");
  // The cooperative copy gives each wave at most one 1 KB piece of the scale rows.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NWV * WBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t scl[SCL];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * ROWS;
  const int64_t ld = K / 2, lsc = K / 32;
  const int KT = K / 128;
  const int ks0 = wave * ST;
  uint8_t* wl = lds + wave * WBYTES;

  // ---- tokens of this wave's segment (lanes whose token is past M, and steps past K,
  // get zeros); tile u holds tokens 16u .. 16u+15 ----
  // Scale words of 4 consecutive steps are one 16-byte load when the segment lies
  // inside the row and rows of scales are 16-byte multiples (K % 512 == 0).
  const bool vec_scales = (K & 511) == 0;
  auto load_words = [&](const uint8_t* rowp, int q, int* dst) {
    const int ks = ks0 + 4 * q;
    if (vec_scales && ks + 4 <= KT) {
      const v4i w4 = *reinterpret_cast<const v4i*>(rowp + ks * 4);
      dst[0] = w4[0]; dst[1] = w4[1]; dst[2] = w4[2]; dst[3] = w4[3];
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) dst[u] = *reinterpret_cast<const int*>(rowp + min(ks + u, KT - 1) * 4);
    }
  };
  v4i t[TT][ST];
  int ts[TT][ST];
  bool tok[TT];
  int64_t trow[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    tok[u] = 16 * u + r < M;
    trow[u] = tok[u] ? 16 * u + r : 0;
  }
  if constexpr (HALF) {
    // Lanes r >= 8 would only hold zeros: let them fetch the next step of token r-8,
    // then rotate each 16-lane row by 8 (DPP row_ror:8) to move it into lanes 0..7.
    const int64_t prow = min(r & 7, M - 1);
#pragma unroll
    for (int s = 0; s < ST; s += 2) {
      const int ks = min(ks0 + s + (r >> 3), KT - 1);
      t[0][s] = *reinterpret_cast<const v4i*>(A + prow * ld + (int64_t)ks * 64 + slot * 16);
    }
  } else {
#pragma unroll
    for (int u = 0; u < TT; ++u)
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const int ks = min(ks0 + s, KT - 1);
        t[u][s] = *reinterpret_cast<const v4i*>(A + trow[u] * ld + (int64_t)ks * 64 + slot * 16);
      }
  }
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int q = 0; q < ST / 4; ++q) load_words(sfA + trow[u] * lsc, q, ts[u] + 4 * q);

  // ---- weight copies: copy i covers rows i*RPI .. i*RPI+RPI-1 of the segment ----
  {
    const int u = lane % UPR, rr = lane / UPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = i * RPI + rr;
      const int gu = u ^ (row & 15);                      // global unit held by LDS unit u
      const int ks = min(ks0 + (gu >> 2), KT - 1);
      const int64_t grow = min(n0 + row, (int64_t)N - 1);
      lds_copy16_nt(B + grow * ld + (int64_t)ks * 64 + (gu & 3) * 16, (lds_void*)(wl + i * 1024));
    }
  }

  // ---- weight scale words: lane (r, slot) needs byte `slot` of word (row, step) ----
  int ws[RG][ST];
  if constexpr (COOP) {
    // The workgroup's rows of scales are one contiguous run of ROWS * K/32 bytes
    // (16-byte aligned: the launcher checks K % 512 == 0 and the base address).
    // Waves copy it in whole-line 1 KB pieces, so every line is requested once.
    const int64_t total = (int64_t)N * lsc;
    const int64_t first = n0 * lsc;
    const int pieces = (int)((min((int64_t)ROWS * lsc, total - first) + 1023) / 1024);
    for (int pc = wave; pc < pieces; pc += NWV) {
      const int64_t off = min(first + pc * 1024 + lane * 16, total - 16);
      lds_copy16(sfB + off, (lds_void*)(scl + pc * 1024));
    }
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int64_t grow = min(n0 + 16 * g + r, (int64_t)N - 1);
#pragma unroll
      for (int q = 0; q < ST / 4; ++q) load_words(sfB + grow * lsc, q, ws[g] + 4 * q);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);          // every load of this wave, copies included
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if constexpr (COOP) {
    __syncthreads();                      // every wave's piece of the scale rows has landed
#pragma unroll
    for (int g = 0; g < RG; ++g) {
#pragma unroll
      for (int q = 0; q < ST / 4; ++q) {
        const int ks = min(ks0 + 4 * q, KT - 4);   // KT % 4 == 0 here; steps past K are masked below
        const v4i w4 = *reinterpret_cast<const v4i*>(scl + (16 * g + r) * lsc + ks * 4);
        ws[g][4 * q] = w4[0]; ws[g][4 * q + 1] = w4[1]; ws[g][4 * q + 2] = w4[2]; ws[g][4 * q + 3] = w4[3];
      }
    }
  }

  if constexpr (HALF) {
#pragma unroll
    for (int s = 0; s < ST; s += 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) t[0][s + 1][e] = __builtin_amdgcn_mov_dpp(t[0][s][e], 0x128, 0xF, 0xF, false);
    }
  }
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const bool ok = tok[u] && ks0 + s < KT;
      ts[u][s] = ok ? (ts[u][s] >> (8 * slot)) & 255 : 127;
      if (!ok) t[u][s] = v4i{0, 0, 0, 0};
    }

  v4f acc[RG][TT];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int row = 16 * g + r;
#pragma unroll
    for (int u = 0; u < TT; ++u) acc[g][u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const v4i w = *reinterpret_cast<const v4i*>(wl + row * SEG + (((s * 4 + slot) ^ (row & 15)) * 16));
      const int wsc = ks0 + s < KT ? (ws[g][s] >> (8 * slot)) & 255 : 127;
#pragma unroll
      for (int u = 0; u < TT; ++u) acc[g][u] = mfma_fp4_16x16<0>(w, t[u][s], acc[g][u], wsc, ts[u][s]);
    }
  }

  // ---- sum the NWV partial tiles in wave order, store D[m][n] ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);   // [NWV][RG * TT][64 lanes][4]
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int u = 0; u < TT; ++u)
      *reinterpret_cast<v4f*>(red + ((wave * RG * TT + g * TT + u) * 64 + lane) * 4) = acc[g][u];
  __syncthreads();
  if (threadIdx.x < RG * TT * 64) {
    const int gu = threadIdx.x >> 6, l = threadIdx.x & 63;   // gu = g * TT + u
    const int g = gu / TT, m = 16 * (gu % TT) + (l & 15);
    v4f v = *reinterpret_cast<const v4f*>(red + (gu * 64 + l) * 4);
#pragma unroll
    for (int w2 = 1; w2 < NWV; ++w2) v += *reinterpret_cast<const v4f*>(red + ((w2 * RG * TT + gu) * 64 + l) * 4);
    const int64_t n = n0 + 16 * g + 4 * (l >> 4);
    if (m < M && n < N) {
      const int avail = (int)min((int64_t)4, (int64_t)N - n);
      store_out4<BF16>(D, (int64_t)m * N + n, avail, v[0], v[1], v[2], v[3]);
    }
  }
}

// Long-K path (K > 16384): KSPLIT waves per 16 weight rows, each streaming a
// contiguous range of K steps with eight 16-byte loads in flight per lane; the
// partial tiles are summed through LDS.
constexpr int KSPLIT = 4;
constexpr int UNROLL = 8;

template <bool BF16>
__global__ void __launch_bounds__(KSPLIT * 64)
fp4_gemv_long_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, void* __restrict__ D) {
  __shared__ float red[KSPLIT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int64_t ld = K / 2, lds_ = K / 32;
  const int KT = K / 128;
  const int ks0 = (int)((int64_t)wave * KT / KSPLIT), ks1 = (int)((int64_t)(wave + 1) * KT / KSPLIT);

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

template <int NJ, int RG, int TT, bool HALF, bool COOP, int NWV>
hipError_t launch_segmented(const FP4Args& a, hipStream_t s) {
  const int64_t g64 = ceil_div(a.N, 16 * RG);
  if (g64 > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)g64), block(NWV * 64);
  if (a.bf16_out)
    hipLaunchKernelGGL((fp4_gemv_kernel<NJ, RG, TT, HALF, COOP, true, NWV>), grid, block, 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  else
    hipLaunchKernelGGL((fp4_gemv_kernel<NJ, RG, TT, HALF, COOP, false, NWV>), grid, block, 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  return hipGetLastError();
}

template <int NJ, int RG, int TT, bool HALF, int NWV>
hipError_t launch_segmented(const FP4Args& a, bool coop, hipStream_t s) {
  return coop ? launch_segmented<NJ, RG, TT, HALF, true, NWV>(a, s) : launch_segmented<NJ, RG, TT, HALF, false, NWV>(a, s);
}

template <int NJ, int RG, int NWV = WAVES>
hipError_t launch_segmented(const FP4Args& a, hipStream_t s) {
  // Cooperative scale copies need 16-byte aligned scale rows and whole segments.
  const bool coop = a.K % (NWV * 4 * NJ * 128) == 0 && (reinterpret_cast<uintptr_t>(a.sfB) & 15) == 0;
  if (a.M <= 8) return launch_segmented<NJ, RG, 1, true, NWV>(a, coop, s);
  if (a.M <= 16) return launch_segmented<NJ, RG, 1, false, NWV>(a, coop, s);
  // A second token tile keeps its tokens in registers: up to 16 steps per wave (K <= 16384).
  if constexpr (NJ <= 4) return launch_segmented<NJ, RG, 2, false, NWV>(a, coop, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool fp4_gemv_fits(int64_t M, int64_t K) { return M >= 1 && (M <= 16 || (M <= 32 && K <= WAVES * 16 * 128)); }

hipError_t launch_fp4_gemv(const FP4Args& a, hipStream_t s) {
  if (!fp4_gemv_fits(a.M, a.K)) return hipErrorInvalidValue;
  const int64_t KT = a.K / 128;
  // Segment of ST = 4*NJ steps per wave, WAVES segments per row: K <= WAVES*ST*128.
  if (KT <= WAVES * 4) return launch_segmented<1, 2>(a, s);     // K <= 4096: 32 rows per workgroup
  if (KT <= WAVES * 8) {                                         // K <= 8192
    if (KT > WAVES * 7) {
      // 7168 < K <= 8192: 4 waves of 16 steps, so each copy reads 1 KB of one row.  Two
      // rows x 512 bytes per copy at this row pitch (4 KB at K = 8192) streamed 3-12%
      // slower.  32 rows per workgroup (half the token re-reads) while ceil(N/32)
      // workgroups take at most two rounds of the CUs and there are more than 8 tokens.
      if (a.M > 8 && ceil_div(a.N, 32) <= 2 * device_cus()) return launch_segmented<4, 2, 4>(a, s);
      return launch_segmented<4, 1, 4>(a, s);
    }
    // 32 rows per workgroup halve the token re-reads (each workgroup reads all M x K
    // tokens), which pays with more than 8 tokens while one workgroup per CU covers N;
    // otherwise 16 rows keep two workgroups, and so more bytes, in flight per CU.
    if (a.M > 8 && ceil_div(a.N, 32) <= device_cus()) return launch_segmented<2, 2>(a, s);
    return launch_segmented<2, 1>(a, s);
  }
  if (KT <= WAVES * 16) return launch_segmented<4, 1>(a, s);    // K <= 16384
  const int64_t g64 = ceil_div(a.N, 16);
  if (g64 > INT32_MAX) return hipErrorInvalidConfiguration;
  const unsigned groups = (unsigned)g64;
  if (a.bf16_out)
    hipLaunchKernelGGL(fp4_gemv_long_kernel<true>, dim3(groups), dim3(KSPLIT * 64), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  else
    hipLaunchKernelGGL(fp4_gemv_long_kernel<false>, dim3(groups), dim3(KSPLIT * 64), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  return hipGetLastError();
}

}  // namespace fp4g
