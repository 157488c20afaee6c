// NVFP4 decode GEMV for gfx950: D[M][N] for 1 <= M <= 32 tokens, the NVFP4 product of
// the GEMM,
//   D[m][n] = gA * gB * sum_k e2m1(A[m,k]) e4m3(sfA[m,k/16]) * e2m1(B[n,k]) e4m3(sfB[n,k/16])
// with one E4M3 scale per 16 K elements (the NVFP4 setup of the NVIDIA/cutlass issue "Add
// FP4 TMA kernel example for Blackwell in CuTe Python DSL", sections "Scale Factor
// Granularity" and "Code Reference").
//
// With a few tokens the weights are the stream that matters.  As in the W4A8 decode
// kernel (the Hopper CUTLASS/CuTe DSL post, section "What changes in the W4A8 builder":
// a 16-token tile for decode), 16 weight rows fill the first operand of the matrix
// instruction and the tokens sit in the other, zero past M: accumulator lane l holds rows
// n = 4*(l/16)+t of one 16-row weight group and token m = l%16 of a 16-token tile.  With
// 17 to 32 tokens a second token tile multiplies the same folded weights, so each weight
// is still read and folded once.
//
// gfx950 has no E4M3-per-16 block scale in its scaled FP4 instruction, so both operands
// are folded exactly to fp16 (nv_fold.hpp) and multiplied by v_mfma_f32_16x16x32_f16
// with fp32 accumulation; the block scales are inside the operands, so the groups add up
// in the accumulator without a per-group fold.  gA*gB multiplies the sum in the epilogue
// as ldexp(acc * gm, ge), as in the GEMM.
//
// gfx950 mapping (K <= 16384), the layout of the W4A8 decode kernel:
//   * one workgroup of 8 waves per RG groups of 16 weight rows; wave w owns the ST
//     consecutive 128-element K groups starting at w*ST for all of the workgroup's rows;
//     its tokens are loaded once and folded once per group for every row group;
//   * lane (r, slot) of a K group holds its 32 consecutive K elements 32*slot..+31 of
//     weight row r (16 bytes) and of token r; instruction q of the group takes elements
//     8q..8q+7 of each lane (four 16x16x32 instructions per group);
//   * the weights reach LDS through 1 KB global->LDS copies of 8 rows x 128 bytes (two
//     groups, whole lines), issued in K-group order, 16-byte units XOR-swizzled by row;
//     the weight scales through dword copies of the rows' scale bytes of the segment;
//   * every load is issued up front, and each row group's next two K groups are folded
//     and multiplied as soon as their copies land (counted vmcnt waits);
//   * the 8 partial tiles of a row group are summed through LDS in wave order, so results
//     are run-to-run identical.
// K groups past K (the last segment of a ragged K) read clamped in-bounds addresses and
// get zero tokens; rows past N read row N-1 and are not stored.
#include "common.hpp"
#include "internal.h"
#include "nv_fold.hpp"

namespace fp4g {
namespace {

constexpr int WAVES = 8;
constexpr int kMaxGroups = 128;             // K <= 16384: 8 waves x 16 groups

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int NJ, int RG, int TT, bool BF16>
__global__ void __launch_bounds__(WAVES * 64)
nvfp4_gemv_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, float gscale, int gexp,
                  void* __restrict__ D) {
  constexpr int ST = 4 * NJ;                 // K groups (64 bytes of E2M1 per row) per wave
  constexpr int NC = RG * ST;                // 1 KB weight copies per wave
  constexpr int SOFF = NC * 1024;            // the weight scales after the weights
  constexpr int SROW = ST * 8;               // scale bytes per row per wave
  constexpr int SDW = RG * 16 * SROW / 4;    // scale dwords per wave
  constexpr int SC = (SDW + 63) / 64;        // dword copies (whole 256-byte copies)
  constexpr int WBYTES = SOFF + SC * 256;
  constexpr int RED = WAVES * RG * TT * 64 * 16;
  static_assert(TT == 1 || TT == 2, "token tiles");
  static_assert(WAVES * WBYTES <= 160 * 1024 && RED <= WAVES * WBYTES, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[WAVES * WBYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, slot = lane >> 4;
  const int KT = K / 128;
  const int ks0 = wave * ST;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RG);
  const int64_t ld = K / 2, lsc = K / 16;
  {  // problem blockIdx.y of a batch stored back to back
    const int64_t b = blockIdx.y;
    A += b * M * ld;
    sfA += b * M * lsc;
    B += b * N * ld;
    sfB += b * N * lsc;
    D = static_cast<uint8_t*>(D) + b * M * N * (BF16 ? 2 : 4);
  }
  uint8_t* wl = lds + wave * WBYTES;

  v4f acc[RG][TT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int u = 0; u < TT; ++u) acc[g][u] = v4f{0.f, 0.f, 0.f, 0.f};

  // One wave's segment.  FULL: all ST groups lie inside K and all rows inside N (every
  // wave but those at a ragged edge), so no address is clamped and no group masked.
  auto segment = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    auto kc = [&](int ks) { return FULL ? ks : min(ks, KT - 1); };
    auto rc = [&](int64_t row) { return FULL ? row : min(row, (int64_t)N - 1); };

    // ---- tokens of the segment: 16 bytes of codes and the two scale bytes of a lane's
    // 32 elements per group.  Lanes r >= M read token 0 (the same lines as lanes r = 0):
    // their columns of the product are never stored. ----
    v4i tc[TT][ST];
    uint32_t tsc[TT][ST];
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int64_t trow = 16 * u + r < M ? 16 * u + r : 0;
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const int ks = kc(ks0 + s);
        tc[u][s] = *reinterpret_cast<const v4i*>(A + trow * ld + (int64_t)ks * 64 + slot * 16);
        // the dword holding this lane's two scale bytes (halves: slots 2j, 2j+1)
        tsc[u][s] = *reinterpret_cast<const uint32_t*>(sfA + trow * lsc + ks * 8 + (slot >> 1) * 4);
      }
    }

    // ---- weight scales: dword j of row `row` (scale bytes 4j..4j+3 of the segment) ->
    // LDS [row][SROW]; entries past the segment repeat the last one inside the padding ----
#pragma unroll
    for (int c = 0; c < SC; ++c) {
      const int i = min(c * 64 + lane, SDW - 1);
      const int row = i / (SROW / 4), j = i % (SROW / 4);
      const int ks = kc(ks0 + j / 2);
      lds_copy4(sfB + rc(n0 + row) * lsc + ks * 8 + (j & 1) * 4, (lds_void*)(wl + SOFF + c * 256));
    }

    // ---- weight copies in K-group order: pair p of groups of row group g is copies
    // (p, g, h), h the 8-row half; the source of copy h is src[g][h] plus p pairs ----
    const uint8_t* src[RG][2];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + (lane >> 3);
        const int gu = (lane & 7) ^ swz8(row);          // global unit held by LDS unit lane & 7
        src[g][h] = B + rc(n0 + 16 * g + row) * ld + (int64_t)ks0 * 64 + gu * 16;
      }
#pragma unroll
    for (int p = 0; p < ST / 2; ++p) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* a = src[g][h] + p * 128;
          if constexpr (!FULL) {
            const int ks = ks0 + 2 * p + (((lane & 7) ^ swz8(8 * h + (lane >> 3))) >> 2);
            if (ks > KT - 1) a -= (int64_t)(ks - (KT - 1)) * 64;
          }
          lds_copy16_nt(a, (lds_void*)(wl + ((p * RG + g) * 2 + h) * 1024));
        }
      }
    }

    // Nothing of the arithmetic below is scheduled among the copies: a token or scale
    // use placed between them would force a wait for every copy issued before it.
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, ST / 2>([&](auto p_c) {
      constexpr int p = decltype(p_c)::value;
      v8h ta[TT][2][4];                               // the pair's folded tokens
      static_for<0, RG>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        __builtin_amdgcn_sched_barrier(0);   // token and scale uses stay after the wait
        wait_vmcnt<RG * ST - 2 * (p * RG + g + 1)>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int s = 2 * p + h;
          if (g == 0) {
#pragma unroll
            for (int u = 0; u < TT; ++u) {
              float p0, p1;
              h2 m0, m1;
              const uint32_t t2 = tsc[u][s] >> (16 * (slot & 1));
              e4m3_split(t2 & 0xFFu, &p0, &m0);
              e4m3_split((t2 >> 8) & 0xFFu, &p1, &m1);
              if (!FULL && ks0 + s >= KT) {           // a group past K adds nothing
                m0 = h2{0, 0};
                m1 = h2{0, 0};
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                uint32_t o[4];
                fold8((uint32_t)tc[u][s][q], q < 2 ? p0 : p1, q < 2 ? m0 : m1, o);
                ta[u][h][q] = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
              }
            }
          }
          const int row = 16 * g + r;
          const v4i x = *reinterpret_cast<const v4i*>(wl + ((p * RG + g) * 2 + (r >> 3)) * 1024 + (r & 7) * 128 +
                                                      (((4 * h + slot) ^ swz8(r)) << 4));
          const uint32_t wsc = *reinterpret_cast<const uint16_t*>(wl + SOFF + row * SROW + s * 8 + slot * 2);
          float p0, p1;
          h2 m0, m1;
          e4m3_split(wsc & 0xFFu, &p0, &m0);
          e4m3_split(wsc >> 8, &p1, &m1);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t o[4];
            fold8((uint32_t)x[q], q < 2 ? p0 : p1, q < 2 ? m0 : m1, o);
            const v8h wv = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
#pragma unroll
            for (int u = 0; u < TT; ++u)
              acc[g][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, ta[u][h][q], acc[g][u], 0, 0, 0);
          }
        }
      });
    });
  };
  if (ks0 + ST <= KT && n0 + 16 * RG <= N) segment(std::true_type{});
  else if (ks0 < KT) segment(std::false_type{});

  // ---- sum the WAVES partial tiles in wave order, scale by gA*gB, store D[m][n] ----
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);   // [WAVES][RG * TT][64 lanes][4]
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
    for (int w2 = 1; w2 < WAVES; ++w2) v += *reinterpret_cast<const v4f*>(red + ((w2 * RG * TT + gu) * 64 + l) * 4);
    const int64_t n = n0 + 16 * g + 4 * (l >> 4);
    if (m < M && n < N) {
      const int avail = (int)min((int64_t)4, (int64_t)N - n);
      store_out4<BF16>(D, (int64_t)m * N + n, avail, __builtin_ldexpf(v[0] * gscale, gexp),
                       __builtin_ldexpf(v[1] * gscale, gexp), __builtin_ldexpf(v[2] * gscale, gexp),
                       __builtin_ldexpf(v[3] * gscale, gexp));
    }
  }
}

template <int NJ, int RG, int TT>
hipError_t launch_tiles(const FP4Args& a, hipStream_t s) {
  const int64_t g64 = ceil_div(a.N, 16 * RG);
  if (g64 > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)g64, (unsigned)a.L), block(WAVES * 64);
  if (a.bf16_out)
    hipLaunchKernelGGL((nvfp4_gemv_kernel<NJ, RG, TT, true>), grid, block, 0, s, (int)a.M, (int)a.N, (int)a.K, a.A,
                       a.sfA, a.B, a.sfB, a.gscale, a.gscale_exp, a.D);
  else
    hipLaunchKernelGGL((nvfp4_gemv_kernel<NJ, RG, TT, false>), grid, block, 0, s, (int)a.M, (int)a.N, (int)a.K,
                       a.A, a.sfA, a.B, a.sfB, a.gscale, a.gscale_exp, a.D);
  return hipGetLastError();
}

template <int NJ, int RG>
hipError_t launch_cfg(const FP4Args& a, hipStream_t s) {
  if (a.M <= 16) return launch_tiles<NJ, RG, 1>(a, s);
  // Two token tiles keep their tokens in registers: up to 8 groups per wave (K <= 8192),
  // which nvfp4_gemv_fits admits.
  if constexpr (NJ <= 2) return launch_tiles<NJ, RG, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool nvfp4_gemv_fits(int64_t M, int64_t K) {
  const int64_t G = K / 128;
  if (M < 1 || K < 128) return false;
  if (M <= 16) return G <= kMaxGroups;
  return M <= 32 && G <= WAVES * 8;                   // two token tiles (launch_cfg)
}

hipError_t launch_nvfp4_gemv(const FP4Args& a, hipStream_t s) {
  if (!nvfp4_gemv_fits(a.M, a.K) || a.K % 128 != 0) return hipErrorInvalidValue;
  const int64_t KT = a.K / 128;
  // Segment of ST = 4*NJ groups per wave, WAVES segments per row: K <= WAVES*ST*128.
  if (KT <= WAVES * 4) return launch_cfg<1, 2>(a, s);     // K <= 4096: 32 rows per workgroup
  if (KT <= WAVES * 8) return launch_cfg<2, 2>(a, s);     // K <= 8192: 32 rows
  return launch_cfg<4, 1>(a, s);                          // K <= 16384: 16 rows
}

}  // namespace fp4g
