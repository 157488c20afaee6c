// NVFP4 GEMM for gfx950: E2M1 operands with one E4M3 scale per 16 K elements and
// one fp32 global scale per operand:
//   D[m][n] = gA * gB * sum_k e2m1(A[m,k]) e4m3(sfA[m,k/16]) * e2m1(B[n,k]) e4m3(sfB[n,k/16])
// The 16-element E4M3 scale granularity is the NVFP4 setup of the NVIDIA/cutlass
// issue "Add FP4 TMA kernel example for Blackwell in CuTe Python DSL" (sections
// "Scale Factor Granularity" and "Code Reference": sf_dtype Float8E4M3FN,
// sf_vec_size 16, so a 128-wide K tile carries 8 scales per row).
//
// gfx950 has no hardware E4M3-per-16 block scale (its scaled MFMA takes E8M0 per
// 32), and e2m1 * e4m3 needs up to 6 significant bits, more than any 8-bit
// float holds.  The exact fold is into fp16 (11 significant bits; every product
// e2m1 * e4m3 lies in [2^-10, 2880], inside fp16's normal range): the scale
// s = 2^e * m (1 <= m < 2, 3 fraction bits) is applied in two exact steps,
// v_cvt_scalef32_pk_f16_fp4 (which widens two codes and multiplies them by the
// power of two of its fp32 scale operand: 2^e) and one v_pk_mul_f16 by (m, m).
// The folded tiles are written to LDS and consumed by v_mfma_f32_16x16x32_f16
// with fp32 accumulation; gA*gB multiplies the accumulator in the epilogue, as an fp32
// significand product and a power of two, ldexp(acc * gm, ge), so that scale pairs whose
// fp32 product would overflow or flush to zero still give every representable D.
//
// Structure: one workgroup per BM x BN tile, 4 or 8 waves of WM x WN; 128 K elements
// (64 packed bytes, two scale dwords) per row per step; packed tiles are prefetched
// into registers two steps ahead; a step reads all its fragments, folds the next step
// while they land, then runs its MFMAs; LDS rows are 256 bytes (128 fp16) with 16-byte
// chunks XOR-swizzled by row.
#include <type_traits>

#include "common.hpp"
#include "internal.h"
#include "nv_fold.hpp"

namespace fp4g {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;            // K elements per step
constexpr int kRowH = kBK * 2;     // 256 bytes of fp16 per LDS row: 16 chunks of 16 bytes

// 16-byte chunk c of LDS row r sits at position c ^ (r & 15): the 16 consecutive rows
// that one MFMA fragment read touches at one logical chunk, and the 4 rows x 4 chunks
// that 16 consecutive threads of the fold write, all land in distinct bank groups.
__device__ __forceinline__ int swz16(int r) { return r & 15; }

// SPLIT: the K steps are cut into S slices of KS steps (the last one shorter); work item
// = tile * S + slice, and the slice's fp32 partial product (without the global scales)
// goes to D = P[L][S][M][N] for launch_scaled_reduce.
template <int BM, int BN, int WM, int WN, bool SPLIT, bool BF16>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
nvfp4_gemm_kernel(int M, int N, int K, int S, int KS, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, float gscale, int gexp,
                  void* __restrict__ D) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int CHUNKS = (BM + BN) * 4;     // 16-byte packed chunks per step
  constexpr int CH = (CHUNKS + NT - 1) / NT; // per thread (the last round may leave threads idle)
  constexpr int FI = WM / 16, FJ = WN / 16;
  static_assert(CHUNKS % NT == 0 || CH == 1, "tile/threads mismatch");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kRowH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int r16 = lane & 15, slot = lane >> 4;
  {  // problem blockIdx.y of a batch stored back to back
    const int64_t b = blockIdx.y;
    A += b * M * (K / 2);
    sfA += b * M * (K / 16);
    B += b * N * (K / 2);
    sfB += b * N * (K / 16);
    D = static_cast<uint8_t*>(D) + b * (SPLIT ? S : 1) * M * N * (SPLIT ? 4 : (BF16 ? 2 : 4));
  }
  const int tiles_n = (N + BN - 1) / BN;
  const int item = (int)blockIdx.x;
  const int tile = SPLIT ? item / S : item, slice = SPLIT ? item % S : 0;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  const int64_t ld = K / 2, lds_ = K / 16;
  const int k0 = SPLIT ? slice * KS : 0;           // this item's steps: k0 .. k0 + KT - 1
  const int KT = SPLIT ? min(KS, K / kBK - k0) : K / kBK;
  if constexpr (SPLIT) D = static_cast<float*>(D) + (int64_t)slice * M * N;

  // Thread chunk q: packed row (A rows first, then B rows), quarter c of its 64 bytes
  // (32 elements, two scales).
  const uint8_t* gsrc[CH];
  const uint8_t* gscl[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int q = min(tid + i * NT, CHUNKS - 1), row = q >> 2, c = q & 3;
    const bool isA = row < BM;
    const int grow = isA ? min(m0 + row, M - 1) : min(n0 + row - BM, N - 1);
    gsrc[i] = (isA ? A : B) + (int64_t)grow * ld + (int64_t)k0 * 64 + c * 16;
    gscl[i] = (isA ? sfA : sfB) + (int64_t)grow * lds_ + k0 * 8 + c * 2;
  }

  // Packed tiles are prefetched two steps ahead into two register buffers (RB = the
  // buffer index, a compile-time constant so the arrays stay in registers); loads
  // past the last step re-read it (in bounds, never used).
  v4i pk[2][CH];
  uint32_t ps[2][CH];
  auto load_global = [&](int kt, auto rb_c) {
    constexpr int RB = decltype(rb_c)::value;
    const int kc = min(kt, KT - 1);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      pk[RB][i] = *reinterpret_cast<const v4i*>(gsrc[i] + (int64_t)kc * 64);
      ps[RB][i] = *reinterpret_cast<const uint16_t*>(gscl[i] + kc * 8);
    }
  };
  auto store_lds = [&](int st, auto rb_c) {
    constexpr int RB = decltype(rb_c)::value;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (CHUNKS % NT != 0 && tid + i * NT >= CHUNKS) break;   // idle thread in a partial round
      const int row = (tid + i * NT) >> 2, c = (tid + i * NT) & 3;
      float p0, p1;
      h2 m0, m1;
      e4m3_split(ps[RB][i] & 0xFFu, &p0, &m0);
      e4m3_split(ps[RB][i] >> 8, &p1, &m1);
#pragma unroll
      for (int d = 0; d < 4; ++d) {   // dword d: elements 8d..8d+7 of the 32
        uint32_t out[4];
        fold8((uint32_t)pk[RB][i][d], d < 2 ? p0 : p1, d < 2 ? m0 : m1, out);
        const int chunk = 4 * c + d;
        *reinterpret_cast<v4i*>(&lds[st][row * kRowH + ((chunk ^ swz16(row)) << 4)]) =
            v4i{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
      }
    }
  };

  v4f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Step kt: all fragments of LDS buffer kt&1 are read into registers; while they land,
  // step kt+1 is folded from register buffer (kt+1)&1 into the other LDS buffer and step
  // kt+3 is fetched into that register buffer; then the step's MFMAs run.
  auto step = [&](int kt, auto rb_c) {
    __syncthreads();
    const int st = kt & 1;
    v8h af[4][FI], bf[4][FJ];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int chunk = 4 * sub + slot;
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int row = wm * WM + i * 16 + r16;
        af[sub][i] = *reinterpret_cast<const v8h*>(&lds[st][row * kRowH + ((chunk ^ swz16(row)) << 4)]);
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int row = BM + wn * WN + j * 16 + r16;
        bf[sub][j] = *reinterpret_cast<const v8h*>(&lds[st][row * kRowH + ((chunk ^ swz16(row)) << 4)]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < KT) {
      store_lds((kt + 1) & 1, rb_c);
      load_global(kt + 3, rb_c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[sub][i], bf[sub][j], acc[i][j], 0, 0, 0);
  };
  const std::integral_constant<int, 0> R0{};
  const std::integral_constant<int, 1> R1{};
  load_global(0, R0);
  load_global(1, R1);
  store_lds(0, R0);
  load_global(2, R0);
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    step(kt, R1);
    step(kt + 1, R0);
  }
  if (kt < KT) step(kt, R1);

#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int n = n0 + wn * WN + j * 16 + r16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + wm * WM + i * 16 + 4 * slot + t;
        if (m < M && n < N) {
          if constexpr (SPLIT) store_out<false>(D, (int64_t)m * N + n, acc[i][j][t]);
          else store_out<BF16>(D, (int64_t)m * N + n, __builtin_ldexpf(acc[i][j][t] * gscale, gexp));
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const FP4Args& a, int64_t S, float* P, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const int64_t KT = a.K / kBK, KS = ceil_div(KT, S);
  const int64_t items = ceil_div(a.N, BN) * ceil_div(a.M, BM) * S;
  if (items > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)items, (unsigned)a.L);
  if (S > 1) {
    hipLaunchKernelGGL((nvfp4_gemm_kernel<BM, BN, WM, WN, true, false>), grid, dim3(NT), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, (int)S, (int)KS, a.A, a.sfA, a.B, a.sfB, a.gscale, a.gscale_exp, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_scaled_reduce(a.L, a.M, a.N, (int)S, P, nullptr, a.gscale, a.gscale_exp, a.D, a.bf16_out, s);
  }
  if (a.bf16_out)
    hipLaunchKernelGGL((nvfp4_gemm_kernel<BM, BN, WM, WN, false, true>), grid, dim3(NT), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, 1, (int)KT, a.A, a.sfA, a.B, a.sfB, a.gscale, a.gscale_exp, a.D);
  else
    hipLaunchKernelGGL((nvfp4_gemm_kernel<BM, BN, WM, WN, false, false>), grid, dim3(NT), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, 1, (int)KT, a.A, a.sfA, a.B, a.sfB, a.gscale, a.gscale_exp, a.D);
  return hipGetLastError();
}

// The tile configuration for L problems of M x N (both paths take it).
bool nv_big_tiles(int64_t L, int64_t M, int64_t N) { return L * ceil_div(M, 128) * ceil_div(N, 128) >= 256; }

}  // namespace

void split_global_scale(float global_a, float global_b, float* m, int* e) {
  int ea = 0, eb = 0;
  const float fa = __builtin_frexpf(global_a, &ea), fb = __builtin_frexpf(global_b, &eb);
  *m = fa * fb;
  *e = ea + eb;
}

hipError_t launch_nvfp4_gemm(const FP4Args& a, hipStream_t s) { return launch_nvfp4_gemm_split(a, 1, nullptr, s); }

int64_t nvfp4_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap) {
  const int64_t KT = K / kBK;
  if (L * M * N == 0 || nvfp4_gemv_fits(M, K) || KT < 2) return 1;
  int64_t smax = KT < kMaxSplits ? KT : kMaxSplits;
  if (cap < smax) smax = cap;
  if (smax < 2) return 1;
  auto slices = [&](int64_t S) { return ceil_div(KT, ceil_div(KT, S)); };   // every slice non-empty
  if (requested > 0) return slices(requested < smax ? requested : smax);
  // Automatic choice: an item streams its K steps at about 0.6 us each plus about 2 us of
  // fixed cost, two items share a CU; the partial products cost a write and a read of
  // L*M*N fp32 per slice at about 4 TB/s.  Problems that fill the chip with 128 x 128
  // tiles are not split; a slice keeps at least 4 steps.
  if (nv_big_tiles(L, M, N)) return 1;
  const int64_t cus = device_cus();
  const int64_t items = L * ceil_div(M, 64) * ceil_div(N, 64);
  int64_t best = 1;
  double best_t = 0;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t sl = slices(S), ks = ceil_div(KT, S);
    if (S > 1 && ks < 4) break;
    const double rounds = (double)ceil_div(items * sl, 2 * cus);
    double t = rounds * ((double)ks * 0.6 + 2.0);
    if (sl > 1) t += (double)(L * M * N) * 4.0 * (double)(2 * sl) / 4.0e6;
    if (S == 1 || t < best_t) { best = sl; best_t = t; }
  }
  return best;
}

hipError_t launch_nvfp4_gemm_split(const FP4Args& a, int64_t splits, float* P, hipStream_t s) {
  if (nvfp4_gemv_fits(a.M, a.K)) return launch_nvfp4_gemv(a, s);         // decode: 16-token tiles
  if (splits > 1 && !P) return hipErrorInvalidValue;
  const int64_t S = splits > 1 ? splits : 1;
  if (nv_big_tiles(a.L, a.M, a.N)) return launch_cfg<128, 128, 64, 64>(a, S, P, s);
  // Small problems: 64 x 64 tiles with 8 waves of 16 x 32, so each SIMD interleaves two
  // waves' folds, LDS traffic and MFMAs (1024^3: 7.1 us, against 8.3 us with 4 waves of
  // 32 x 32, which read a third less from LDS but fold with half as many threads).
  return launch_cfg<64, 64, 16, 32>(a, S, P, s);
}

}  // namespace fp4g
