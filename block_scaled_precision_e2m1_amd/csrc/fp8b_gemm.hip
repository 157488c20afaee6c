// FP8 blockwise-scaled GEMM for gfx950: E4M3 operands with one fp32 scale per row
// per 128-element K group,
//   D[m][n] = sum_g sA[m][g] * sB[n][g] * sum_{k in group g} e4m3(A[m][k]) * e4m3(B[n][k]).
// This is the FP8 blockwise GEMM that the NVIDIA/cutlass issue "Add FP4 TMA kernel
// example for Blackwell in CuTe Python DSL" takes as its starting point ("What
// Works", and "Scale Factor Granularity": FP8 uses a granularity of 128 along K).
//
// gfx950 design:
//   * workgroup tile 256 x 128 (8 waves in a 4 x 2 grid of 64 x 64) when such tiles
//     fill the CUs, else 128 x 128 (8 waves in a 2 x 4 grid of 64 x 32); a stage is
//     one 128-element group: 128 FP8 bytes (one cache line) per row of A and of B, and
//     the group's fp32 scales;
//   * stages reach LDS through global->LDS copies (global_load_lds_dwordx4 for the
//     operands, _dword for the scales) into a 3- or 4-slot ring, waited for with counted
//     vmcnt and one barrier per stage; 16-byte chunks are XOR-swizzled by row so the
//     MFMA-layout ds_read_b128 is free of bank conflicts;
//   * a group's product is two v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 x FP8, unit
//     E8M0 scales) per 32 x 32 block into partial-sum registers; the fp32 accumulator then
//     takes it times sA[m][g] * sB[n][g] (no FP8 value can absorb an fp32 scale
//     exactly, so the scaling is a VALU multiply-add per element and group);
//   * B is the first MFMA operand, so the accumulator holds D^T: a lane owns one m
//     and four consecutive n per register quad, stored as one 8- or 16-byte write.
#include <type_traits>

#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int FBM = 128, FBN = 128;
constexpr int FSTAGES = 4;
constexpr int F_A = FBM * 128;              // FP8 bytes of A per stage (16 KB)
constexpr int F_B = FBN * 128;              // FP8 bytes of B per stage (16 KB)
constexpr int F_SA = F_A + F_B;             // sA: 128 fp32
constexpr int F_SB = F_SA + FBM * 4;        // sB: 128 fp32
constexpr int F_STAGE = F_SB + FBN * 4;
static_assert(FSTAGES * F_STAGE <= 160 * 1024, "LDS budget");
// Copies per wave per stage with W waves: 16/W of A and of B (1 KB each), one scale copy.
template <int W>
constexpr int f_loads() { return 2 * (16 / W) + 1; }
static_assert((FSTAGES - 2) * f_loads<4>() < 64, "vmcnt range");

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// NWN waves along N (2 or 4): 2*NWN waves of 64 x (128/NWN).
template <int NWN, bool BF16>
__global__ void __launch_bounds__(2 * NWN * 64)
fp8b_gemm_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
                 const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D) {
  constexpr int W = 2 * NWN, CPW = 16 / W, WN = FBN / NWN, FJ = WN / 32;
  constexpr int F_LOADS = f_loads<W>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[FSTAGES * F_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int hi = lane >> 5, r32 = lane & 31;

  // Tile order: consecutive ids go to the 8 XCDs in turn; regroup so each XCD owns a
  // contiguous band of tiles (shared A and B panels in its L2).
  const int tiles_m = (M + FBM - 1) / FBM, tiles_n = (N + FBN - 1) / FBN;
  const int T = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((T & 7) == 0) lin = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int m0 = (lin / tiles_n) * FBM, n0 = (lin % tiles_n) * FBN;
  const int G = K / 128;

  // ---- copy sources: copy c (0..15) of an operand covers rows 8c .. 8c+7 ----
  const uint8_t* ga[CPW];
  const uint8_t* gb[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = wave * CPW + i;
    const int row = 8 * c + (lane >> 3), u = lane & 7;
    ga[i] = A + (int64_t)min(m0 + row, M - 1) * K + ((u ^ swz8(row)) << 4);
    gb[i] = B + (int64_t)min(n0 + row, N - 1) * K + ((u ^ swz8(row)) << 4);
  }
  // Scale copy z = wave % 4 fetches 64 scales -- sA rows 0..63 / 64..127, sB rows 0..63 /
  // 64..127; with 8 waves, waves z and z+4 write the same bytes to the same place.
  const int sz = wave & 3;
  const int srow = 64 * (sz & 1) + lane;
  const float* gs = (sz < 2) ? sA + (int64_t)min(m0 + srow, M - 1) * G : sB + (int64_t)min(n0 + srow, N - 1) * G;
  const int ls = ((sz < 2) ? F_SA : F_SB) + 256 * (sz & 1);

  auto issue = [&](int g) {
    const int gc = min(g, G - 1);                  // past the end: re-read the last group
    uint8_t* base = smem + (g % FSTAGES) * F_STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) lds_copy16(ga[i] + (int64_t)gc * 128, (lds_void*)(base + (wave * CPW + i) * 1024));
#pragma unroll
    for (int i = 0; i < CPW; ++i)
      lds_copy16(gb[i] + (int64_t)gc * 128, (lds_void*)(base + F_A + (wave * CPW + i) * 1024));
    lds_copy4(gs + gc, (lds_void*)(base + ls));
  };

  v16f acc[2][FJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v16f{};
  const int unit = 0x7F7F7F7F;

#pragma unroll
  for (int p = 0; p < FSTAGES - 1; ++p) issue(p);

  // Software pipeline: the MFMAs of group g run while the VALU folds group g-1's
  // partial sums (and their scales, read from LDS during iteration g-1) into the
  // accumulator, so the matrix pipe and the vector ALU overlap.
  v16f part[2][2][FJ];                              // [buffer][i][j]
  float sa_r[2][2];                                 // [buffer][i]: sA of the lane's row
  v4f sb_r[2][FJ][4];                               // [buffer][j][q]: sB of the lane's 16 columns
  auto read_scales = [&](const uint8_t* base, int buf) {
    const float* ssa = reinterpret_cast<const float*>(base + F_SA);
    const float* ssb = reinterpret_cast<const float*>(base + F_SB);
#pragma unroll
    for (int i = 0; i < 2; ++i) sa_r[buf][i] = ssa[wm * 64 + i * 32 + r32];
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sb_r[buf][j][q] = *reinterpret_cast<const v4f*>(ssb + wn * WN + j * 32 + 8 * q + 4 * hi);
  };
  // part[buf][i][j] holds D^T: element t of lane (hi, r32) is n = 32j + 8(t/4) + 4hi + t%4,
  // m = 32i + r32 of the wave tile.
  auto fold = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][4 * q + e] =
                __builtin_fmaf(part[buf][i][j][4 * q + e], sa_r[buf][i] * sb_r[buf][j][q][e], acc[i][j][4 * q + e]);
  };
  auto group = [&](int g, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    // Group g is complete once only groups g+1 .. g+FSTAGES-2 are in flight; the barrier
    // publishes every wave's copies and frees slot (g-1) % FSTAGES.
    wait_vmcnt<(FSTAGES - 2) * F_LOADS>();
    barrier_lds();
    issue(g + FSTAGES - 1);
    const uint8_t* base = smem + (g % FSTAGES) * F_STAGE;
    read_scales(base, BUF);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c0 = 4 * kk + 2 * hi;              // this lane's 32 bytes: chunks c0, c0+1
      v8i af[2], bf[FJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + r32;
        const v4i x0 = *reinterpret_cast<const v4i*>(base + row * 128 + ((c0 ^ swz8(row)) << 4));
        const v4i x1 = *reinterpret_cast<const v4i*>(base + row * 128 + (((c0 + 1) ^ swz8(row)) << 4));
        af[i] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int row = wn * WN + j * 32 + r32;
        const v4i x0 = *reinterpret_cast<const v4i*>(base + F_A + row * 128 + ((c0 ^ swz8(row)) << 4));
        const v4i x1 = *reinterpret_cast<const v4i*>(base + F_A + row * 128 + (((c0 + 1) ^ swz8(row)) << 4));
        bf[j] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      // The group's MFMAs at raised wave priority, the fold at normal priority: the two
      // waves sharing a SIMD then tend to run opposite phases (one multiplying, one
      // folding) between barriers (4096^3: 149 against 152 us on the same box).
      if (kk == 0) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          part[BUF][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bf[j], af[i], kk == 0 ? v16f{} : part[BUF][i][j], kFmtFp8, kFmtFp8, 0, unit, 0, unit);
    }
    __builtin_amdgcn_s_setprio(0);
    if (g > 0) fold(BUF ^ 1);
  };

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

  // Epilogue: lane (hi, r32) of block (i, j) owns row m = 32i + r32 and, for q = 0..3,
  // the four consecutive columns n = 32j + 8q + 4hi + 0..3.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + i * 32 + r32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * hi;
        if (n < N)
          store_out4<BF16>(D, (int64_t)m * N + n, N - n, acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]);
      }
  }
}

// ---- 256 x 128 tiles -----------------------------------------------------------------
// Twice the work per barrier and a third less LDS traffic per FLOP than the 128 x 128
// tile: 8 waves of 64 x 64 in a 4 x 2 grid, two per SIMD. An operand stage is 48 KB, so
// the ring holds three; each group's scales go to a ring of four slots of their own, so
// they outlive the group's operand slot by one group and the fold can read them one
// group late. Each wave keeps one set of partial sums: the fold of group g-1 into the
// accumulator runs block by block, each block's fold just before the first MFMA of group
// g that overwrites the block, so the next block's fold issues while that MFMA runs.
constexpr int GBM = 256, GBN = 128;
constexpr int GSTAGES = 3, GSCALE_SLOTS = 4;
constexpr int G_A = GBM * 128;                      // 32 KB of A
constexpr int G_STAGE = G_A + GBN * 128;            // + 16 KB of B
constexpr int G_SCALES = GSTAGES * G_STAGE;         // scale ring: sA (1 KB) then sB (512 B)
constexpr int G_SSLOT = (GBM + GBN) * 4;
constexpr int G_LDS = G_SCALES + GSCALE_SLOTS * G_SSLOT;
static_assert(G_LDS <= 160 * 1024, "LDS budget");
// Per wave per stage: 4 copies of A, 2 of B (1 KB each) and one 256-byte scale copy.
constexpr int G_LOADS = 4 + 2 + 1;
static_assert((GSTAGES - 2) * G_LOADS < 64, "vmcnt range");

template <bool BF16>
__global__ void __launch_bounds__(512)
fp8b_gemm_big_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sA,
                     const uint8_t* __restrict__ B, const float* __restrict__ sB, void* __restrict__ D) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[G_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;           // 4 x 2 waves of 64 x 64
  const int hi = lane >> 5, r32 = lane & 31;

  const int tiles_m = (M + GBM - 1) / GBM, tiles_n = (N + GBN - 1) / GBN;
  const int T = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((T & 7) == 0) lin = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  // Consecutive ids go to the 8 XCDs in turn: regroup so each XCD owns a contiguous
  // range of ids. Then walk groups of 4 tile rows column by column, so the 32 tiles
  // that one XCD runs at once form a 4 x 8 block: per 128-element group they share 4 A
  // and 8 B slices in that XCD's L2 instead of 1 and 32 (4096^3: 139 against 291 MB
  // fetched per launch, 115 against 117.5 us on the same box).
  const int grp = lin / (4 * tiles_n), first = 4 * grp;
  const int gm = min(tiles_m - first, 4), r = lin - grp * 4 * tiles_n;
  const int m0 = (first + r % gm) * GBM, n0 = (r / gm) * GBN;
  const int G = K / 128;

  // Copy c of an operand covers its rows 8c .. 8c+7: A copies 4w .. 4w+3, B copies 2w, 2w+1.
  const uint8_t* ga[4];
  const uint8_t* gb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3), u = lane & 7;
    ga[i] = A + (int64_t)min(m0 + row, M - 1) * K + ((u ^ swz8(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + (lane >> 3), u = lane & 7;
    gb[i] = B + (int64_t)min(n0 + row, N - 1) * K + ((u ^ swz8(row)) << 4);
  }
  // Six 64-row scale pieces (sA rows 0..255, sB rows 0..127); waves 6 and 7 repeat pieces
  // 0 and 1 (same bytes to the same place), so every wave issues the same number of copies.
  const int piece = wave < 6 ? wave : wave - 6;
  const int srow = 64 * (piece & 3) + lane;
  const float* gs = piece < 4 ? sA + (int64_t)min(m0 + srow, M - 1) * G : sB + (int64_t)min(n0 + srow, N - 1) * G;
  const int ls = 256 * piece;                        // sA pieces at 0..1023, sB at 1024..1535

  auto issue = [&](int g) {
    const int gc = min(g, G - 1);                    // past the end: re-read the last group
    uint8_t* base = smem + (g % GSTAGES) * G_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(ga[i] + (int64_t)gc * 128, (lds_void*)(base + (4 * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_copy16(gb[i] + (int64_t)gc * 128, (lds_void*)(base + G_A + (2 * wave + i) * 1024));
    lds_copy4(gs + gc, (lds_void*)(smem + G_SCALES + (g % GSCALE_SLOTS) * G_SSLOT + ls));
  };
  // The lane's 32 bytes of a 64-element K half: 16-byte chunks c0 and c0+1 of the row.
  auto frag = [&](const uint8_t* base, int row, int c0) {
    const v4i x0 = *reinterpret_cast<const v4i*>(base + row * 128 + ((c0 ^ swz8(row)) << 4));
    const v4i x1 = *reinterpret_cast<const v4i*>(base + row * 128 + (((c0 + 1) ^ swz8(row)) << 4));
    return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };

  // acc[i][j] and part[i][j] hold D^T of the wave's 32 x 32 block (i, j): element t of
  // lane (hi, r32) is n = 32j + 8(t/4) + 4hi + t%4, m = 32i + r32 of the wave tile.
  v16f acc[2][2], part[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  const int unit = 0x7F7F7F7F;
  float sav[2];                                      // sA of the lane's two rows, group g-1
  v4f sbv[2][4];                                     // sB of the lane's 32 columns, group g-1
  auto read_scales = [&](int g) {
    const float* ssa = reinterpret_cast<const float*>(smem + G_SCALES + (g % GSCALE_SLOTS) * G_SSLOT);
#pragma unroll
    for (int i = 0; i < 2; ++i) sav[i] = ssa[wm * 64 + i * 32 + r32];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sbv[j][q] = *reinterpret_cast<const v4f*>(ssa + GBM + wn * 64 + j * 32 + 8 * q + 4 * hi);
  };
  auto fold_block = [&](int i, int j) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[i][j][4 * q + e] = __builtin_fmaf(part[i][j][4 * q + e], sav[i] * sbv[j][q][e], acc[i][j][4 * q + e]);
  };

#pragma unroll
  for (int p = 0; p < GSTAGES - 1; ++p) issue(p);

  for (int g = 0; g < G; ++g) {
    // Group g is complete once only group g+1's copies are in flight; the barrier
    // publishes every wave's copies and frees operand slot (g-1) % 3 and scale slot
    // (g-2) % 4 for the copies of group g+2.
    wait_vmcnt<(GSTAGES - 2) * G_LOADS>();
    barrier_lds();
    issue(g + GSTAGES - 1);
    const uint8_t* base = smem + (g % GSTAGES) * G_STAGE;
    if (g > 0) read_scales(g - 1);
    v8i af0[2], bf0[2], af1[2], bf1[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) af0[i] = frag(base, wm * 64 + i * 32 + r32, 2 * hi);
#pragma unroll
    for (int j = 0; j < 2; ++j) bf0[j] = frag(base + G_A, wn * 64 + j * 32 + r32, 2 * hi);
    // The scheduling barriers keep this order: left alone, the compiler puts all four
    // folds ahead of the first MFMA (4096^3: 119 against 123 us on the same box).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = b >> 1, j = b & 1;
      if (g > 0) fold_block(i, j);
      part[i][j] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf0[j], af0[i], v16f{}, kFmtFp8, kFmtFp8, 0, unit, 0, unit);
      if (b == 1) {                                  // second K half's fragments, read mid-way
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) af1[ii] = frag(base, wm * 64 + ii * 32 + r32, 4 + 2 * hi);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) bf1[jj] = frag(base + G_A, wn * 64 + jj * 32 + r32, 4 + 2 * hi);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        part[i][j] =
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf1[j], af1[i], part[i][j], kFmtFp8, kFmtFp8, 0, unit, 0, unit);
  }
  if (G > 0) {
    read_scales(G - 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) fold_block(b >> 1, b & 1);
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + i * 32 + r32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + j * 32 + 8 * q + 4 * hi;
        if (n < N)
          store_out4<BF16>(D, (int64_t)m * N + n, N - n, acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]);
      }
  }
}

hipError_t launch_big(const Fp8bArgs& a, int64_t tiles, hipStream_t s) {
  if (a.bf16_out)
    hipLaunchKernelGGL((fp8b_gemm_big_kernel<true>), dim3((unsigned)tiles), dim3(512), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sA, a.B, a.sB, a.D);
  else
    hipLaunchKernelGGL((fp8b_gemm_big_kernel<false>), dim3((unsigned)tiles), dim3(512), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sA, a.B, a.sB, a.D);
  return hipGetLastError();
}

template <int NWN>
hipError_t launch_nwn(const Fp8bArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.M, FBM) * ceil_div(a.N, FBN);
  if (tiles > INT32_MAX) return hipErrorInvalidConfiguration;
  if (a.bf16_out)
    hipLaunchKernelGGL((fp8b_gemm_kernel<NWN, true>), dim3((unsigned)tiles), dim3(2 * NWN * 64), 0, s, (int)a.M,
                       (int)a.N, (int)a.K, a.A, a.sA, a.B, a.sB, a.D);
  else
    hipLaunchKernelGGL((fp8b_gemm_kernel<NWN, false>), dim3((unsigned)tiles), dim3(2 * NWN * 64), 0, s, (int)a.M,
                       (int)a.N, (int)a.K, a.A, a.sA, a.B, a.sB, a.D);
  return hipGetLastError();
}

}  // namespace

// 8 waves of 64 x 32: about 200 registers, so two waves share a SIMD and one wave's fold runs
// beside another's MFMAs (4096^3: 145 us against 150 us with 4 waves of 64 x 64; same bits).
// 256 x 128 tiles when they alone fill the CUs (4096^3: 119 us against 147 us with
// 128 x 128 tiles on the same box); otherwise 128 x 128, which keeps more CUs busy.
hipError_t launch_fp8b_gemm(const Fp8bArgs& a, hipStream_t s) {
  const int64_t big = ceil_div(a.M, GBM) * ceil_div(a.N, GBN);
  if (big >= device_cus() && big <= INT32_MAX) return launch_big(a, big, s);
  return launch_nwn<4>(a, s);
}

}  // namespace fp4g
