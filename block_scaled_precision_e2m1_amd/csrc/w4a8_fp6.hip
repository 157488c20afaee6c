// W4A8 GEMM over weights re-encoded as FP6 once, when they are loaded (gfx950).
//
// The product is that of w4a8_gemm,
//   D[m][n] = sa[m] * sum_g sB[n][g] * sum_{k in g} e4m3(A[m][k]) * int4(B[n][k]),
// groups of 128 K elements.  The Hopper CUTLASS/CuTe DSL post (section "The W4A8 kernel:
// the same four definitions, with the operands swapped") makes the INT4 -> FP8 conversion
// cheap by re-encoding and re-ordering the weights at load time.  On gfx950 the
// re-encoding can remove the conversion altogether: every INT4 value q in -8..7 is exact
// in the FP6 format E3M2 (sign, 3 exponent bits with bias 3, 2 mantissa bits:
// |q| = 2^(e-3) * (1 + m/4)), and the scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies an E3M2 operand by an E4M3 operand at the
// FP8 rate.  One instruction per 128-K group then gives the group's exact integer-weight
// products, half the instructions of the two-part split that the INT4 kernels use, and no
// VALU work on the weights.  Measured on gfx950: its results equal those of the FP8 x FP8
// instruction on E4M3(q) weights bit for bit (the same truncated in-instruction sum), and
// FP6 lane (r, slot)'s element e (bits 6e .. 6e+5 of the lane's six dwords) pairs with
// the FP8 element of K = 64*(slot & 1) + 16*(slot >> 1) + e + (e < 16 ? 0 : 16), where an
// FP8 lane of slot s holds K = 32s .. 32s+31.
//
// Re-pack.  Blocks of 32 weight rows g32 and K groups kg, 3072 bytes each:
//   Bp6[g32][kg]: bytes    0..1023  lane l's dwords 0-3 for rows 32*g32 + 0..15,
//                 bytes 1024..2047  the same for rows 32*g32 + 16..31,
//                 bytes 2048..3071  lane l's dwords 4-5 of the first half, then of the
//                                   second (16 bytes per lane),
// lane l = 16*slot + r holding row r of its half at the K order above (K offset 128*kg).
// Rows past N are zero codes.  The group scales are w4a8_prepack's Sp [KG][16*ceil(N/16)]
// fp32 (rows past N 0).
//
// Kernel.  Tile 64 tokens x 128 weight rows, 8 waves in a 2 x 4 grid: wave w owns tokens
// 32*(w & 1) .. +31 (two FP8 operands, the instruction's first) and weight rows
// 32*(w >> 1) .. +31 (two FP6 operands, its second), so a lane's four accumulators are
// four tokens of one weight row and take one group scale.  A stage is one K group: 64 x
// 128 B of activations (16-byte chunks XOR-swizzled by row), 4 x 3 KB of FP6 weights and
// the tile's 128 scales, copied HBM -> LDS by global_load_lds (three 1 KB copies per wave)
// into a 6-slot ring with counted waits and one barrier per group.  The barrier of group
// g certifies stage g+1, whose fragments are read into a second register set while group
// g's 4 instructions per wave run; each goes to fresh registers (VGPR form: this file is
// built with the matrix results in VGPRs) and is folded into the fp32 accumulator times
// sB[n][g] while the next group's instructions run.  The epilogue multiplies by sa[m].
//
// What bounds it (256 x 8192 x 8192, measured): the copies.  Each copy instruction costs
// the texture path about 16 cycles for its 64 lanes, so the 24 copies of a group take
// about as long as its 256 cycles of matrix work per SIMD even from L2, and the weights,
// read once from HBM and shared by the four token tiles of a panel, arrive at about
// 2 TB/s.  A copy-only version of the kernel takes 28 us of its 31.  A deeper ring (6 slots
// instead of 4) gained 2 us, but one more group of lead in the same slots gained nothing;
// K-major weight blocks and a ninth wave gathering the next groups' weight lines into L2
// gained nothing or lost.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int F6_BM = 64;                  // tokens per tile
constexpr int F6_BN = 128;                 // weight rows per tile (4 waves x 32)
constexpr int F6_STAGES = 6;
constexpr int F6_T_OFF = 0;                // activations: 64 rows x 128 B
constexpr int F6_W_OFF = F6_BM * 128;      // weights: 4 row quarters x 3072 B
constexpr int F6_S_OFF = F6_W_OFF + 4 * 3072;   // scales: 4 quarters x 1 KB (128 B used)
constexpr int F6_STAGE = F6_S_OFF + 4 * 1024;
constexpr int F6_LOADS = 3;                // copies per wave per stage
static_assert(F6_STAGES * F6_STAGE <= 160 * 1024, "LDS budget");
static_assert((F6_STAGES - 2) * F6_LOADS < 64, "vmcnt range");

constexpr int kFmtE3M2 = 3;
// The activation copies take a 32-bit lane offset of up to 127 rows: 128 * K < 2^31.
constexpr int64_t kFp6MaxK = int64_t(1) << 23;

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// E3M2 codes of the two's-complement nibbles, 6 bits each at bits 6*(n & 7): nibbles
// 0..7 (values 0..7) in kE3M2Lo, nibbles 8..15 (values -8..-1) in kE3M2Hi.
constexpr uint64_t kE3M2Lo = 0x00ull | 0x0Cull << 6 | 0x10ull << 12 | 0x12ull << 18 | 0x14ull << 24 |
                             0x15ull << 30 | 0x16ull << 36 | 0x17ull << 42;
constexpr uint64_t kE3M2Hi = 0x38ull | 0x37ull << 6 | 0x36ull << 12 | 0x35ull << 18 | 0x34ull << 24 |
                             0x32ull << 30 | 0x30ull << 36 | 0x2Cull << 42;

__device__ __forceinline__ uint32_t e3m2_of_nibble(uint32_t n) {
  return (uint32_t)(((n < 8 ? kE3M2Lo : kE3M2Hi) >> (6 * (n & 7))) & 63u);
}

// One thread per (g32, kg, lane): both 16-row halves of the lane.
__global__ void __launch_bounds__(256)
w4a8_prepack_fp6_kernel(int64_t units, int N, int G, int64_t ld, const uint8_t* __restrict__ B,
                        uint8_t* __restrict__ Bp) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63), r = l & 15, slot = l >> 4;
    const int64_t blk = u >> 6;                      // g32 * G + kg
    const int kg = (int)(blk % G);
    const int64_t g32 = blk / G;
    uint32_t w[2][6];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = 32 * g32 + 16 * h + r;
#pragma unroll
      for (int d = 0; d < 6; ++d) w[h][d] = 0;
      if (row < N) {
        // elements 0..15 at K offset k0, 16..31 at k0 + 32: two runs of 8 bytes
        const int k0 = 128 * kg + 64 * (slot & 1) + 16 * (slot >> 1);
        const uint8_t* src = B + row * ld + k0 / 2;
        const uint64_t lo = *reinterpret_cast<const uint64_t*>(src);
        const uint64_t hi = *reinterpret_cast<const uint64_t*>(src + 16);
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const uint32_t n = (uint32_t)(((e < 16 ? lo : hi) >> (4 * (e & 15))) & 15u);
          const uint32_t c = e3m2_of_nibble(n);
          const int bit = 6 * e;
          w[h][bit / 32] |= c << (bit % 32);
          if (bit % 32 > 26) w[h][bit / 32 + 1] |= c >> (32 - bit % 32);
        }
      }
    }
    uint8_t* dst = Bp + blk * 3072;
    *reinterpret_cast<v4i*>(dst + l * 16) = v4i{(int)w[0][0], (int)w[0][1], (int)w[0][2], (int)w[0][3]};
    *reinterpret_cast<v4i*>(dst + 1024 + l * 16) = v4i{(int)w[1][0], (int)w[1][1], (int)w[1][2], (int)w[1][3]};
    *reinterpret_cast<v4i*>(dst + 2048 + l * 16) = v4i{(int)w[0][4], (int)w[0][5], (int)w[1][4], (int)w[1][5]};
  }
}

template <bool BF16>
__global__ void __launch_bounds__(512, 1)
w4a8f6_gemm_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const float* __restrict__ sa,
                   const uint8_t* __restrict__ Bp, const float* __restrict__ Sp, void* __restrict__ D) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F6_STAGES * F6_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = wave & 1, rg = wave >> 1;         // token half, weight-row quarter
  const int r = lane & 15, slot = lane >> 4;

  // Tile order: the token tiles of one weight panel are adjacent (they share it in L2);
  // consecutive ids go to the 8 XCDs in turn and are regrouped per XCD.
  const int tiles_m = (M + F6_BM - 1) / F6_BM, tiles_n = (N + F6_BN - 1) / F6_BN;
  const int T = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((T & 7) == 0) lin = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int m0 = (lin % tiles_m) * F6_BM, n0 = (lin / tiles_m) * F6_BN;
  const int G = K / 128;
  const int G32 = (N + 31) / 32;
  const int64_t Np = 16 * (int64_t)((N + 15) / 16);

  // ---- copy sources: a wave-uniform base advanced per group plus a fixed 32-bit lane
  // offset (64 * K < 2^31).  Per stage each wave copies 8 activation rows (1 KB); in
  // its weight quarter the even wave copies both halves' dwords 0-3 (2 x 1 KB), the odd
  // wave the dwords 4-5 (1 KB) and the quarter's 32 scales. ----
  const uint8_t* ua = A + (int64_t)m0 * K;
  uint32_t va;
  {
    const int row = 8 * wave + (lane >> 3), u = lane & 7;
    va = (uint32_t)((min(m0 + row, M - 1) - m0) * K + ((u ^ swz8(row)) << 4));
  }
  const uint8_t* ub = Bp + (int64_t)min(n0 / 32 + rg, G32 - 1) * G * 3072 + (tg ? 2048 : 0);
  const uint32_t vb = (uint32_t)lane * 16;
  // scales: 16 bytes (4 rows) per lane, lanes 8..63 repeating lanes 0..7 (Sp is 16-byte
  // aligned and Np a multiple of 16)
  const int64_t srow0 = min((int64_t)n0 + 32 * rg, Np - 4);
  const uint8_t* us = reinterpret_cast<const uint8_t*>(Sp) + srow0 * 4;
  const uint32_t vs = (uint32_t)(min(srow0 + 4 * (lane & 7), Np - 4) - srow0) * 4;

  // The second copy: the other half's dwords 0-3 (even wave) or the quarter's scales
  // (odd wave), chosen once here so the copies carry no branch.
  const uint8_t* u2 = tg ? us : ub + 1024;
  const int64_t step2 = tg ? Np * 4 : 3072;
  const uint32_t v2 = tg ? vs : vb;
  const int w1 = F6_W_OFF + rg * 3072 + (tg ? 2048 : 0);
  const int w2 = tg ? F6_S_OFF + rg * 1024 : w1 + 1024;

  auto issue = [&](int g, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    const int gc = min(g, G - 1);                  // past the end: re-read the last group
    uint8_t* base = smem + SLOT * F6_STAGE;
    lds_copy16(ua + (int64_t)gc * 128 + va, (lds_void*)(base + F6_T_OFF + wave * 1024));
    lds_copy16(ub + (int64_t)gc * 3072 + vb, (lds_void*)(base + w1));
    lds_copy16(u2 + (int64_t)gc * step2 + v2, (lds_void*)(base + w2));
  };

  // acc[h][i]: weight half h (16 rows), token block i (16 tokens); lane (slot, r) element t
  // holds token 32tg + 16i + 4slot + t and weight row 32rg + 16h + r.
  v4f acc[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[h][i] = v4f{0.f, 0.f, 0.f, 0.f};
  const int unit = 0x7F7F7F7F;

  static_for<0, F6_STAGES - 1>([&](auto p) { issue(p, p); });

  // One group's LDS fragments: the wave's two FP6 operands and their two scales, and its
  // 32 tokens.  Two register sets: the next group's are read while this group's multiply.
  struct Frag { v8i w[2]; float s[2]; v8i a[2]; };
  Frag fr[2];
  // The fold before group 0 adds part[1] * sc[1] = 0 * 0.
  v4f part[2][2][2];
  float sc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 2; ++i) part[1][h][i] = v4f{0.f, 0.f, 0.f, 0.f};
  auto load = [&](auto slot_c, auto set_c) {
    constexpr int SLOT = decltype(slot_c)::value, SET = decltype(set_c)::value;
    const uint8_t* base = smem + SLOT * F6_STAGE;
    Frag& f = fr[SET];
    const uint8_t* wb = base + F6_W_OFF + rg * 3072 + lane * 16;
    const v4i w0 = *reinterpret_cast<const v4i*>(wb);
    const v4i w1 = *reinterpret_cast<const v4i*>(wb + 1024);
    const v4i wh = *reinterpret_cast<const v4i*>(wb + 2048);
    f.w[0] = v8i{w0[0], w0[1], w0[2], w0[3], wh[0], wh[1], 0, 0};
    f.w[1] = v8i{w1[0], w1[1], w1[2], w1[3], wh[2], wh[3], 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f.s[h] = *reinterpret_cast<const float*>(base + F6_S_OFF + rg * 1024 + (16 * h + r) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * tg + 16 * i + r;
      const v4i a0 = *reinterpret_cast<const v4i*>(base + F6_T_OFF + row * 128 + (((2 * slot) ^ swz8(row)) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(base + F6_T_OFF + row * 128 + (((2 * slot + 1) ^ swz8(row)) << 4));
      f.a[i] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  };
  auto fold = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[h][i][t] = __builtin_fmaf(part[buf][h][i][t], sc[buf][h], acc[h][i][t]);
  };

  // Group g in ring slot J = g % F6_STAGES (BUF = g & 1): stage g+1 has landed and stage
  // g's fragments are in set BUF.  The copies, the next group's LDS reads and the
  // previous group's fold go between the 4 MFMAs.
  auto group = [&](int g, auto j_c) {
    constexpr int J = decltype(j_c)::value, BUF = J & 1;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(F6_STAGES - 3) * F6_LOADS>();
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    issue(g + F6_STAGES - 1, std::integral_constant<int, (J + F6_STAGES - 1) % F6_STAGES>{});
    load(std::integral_constant<int, (J + 1) % F6_STAGES>{}, std::integral_constant<int, BUF ^ 1>{});
    const Frag& f = fr[BUF];
    sc[BUF][0] = f.s[0];
    sc[BUF][1] = f.s[1];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        part[BUF][h][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f.a[i], f.w[h], v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp8, kFmtE3M2, 0, unit, 0, unit);
    fold(BUF ^ 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // three LDS reads
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global -> LDS copy
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // stage 0 landed: its fragments into set 0
  wait_vmcnt<(F6_STAGES - 2) * F6_LOADS>();
  barrier_lds();
  load(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  static_assert(F6_STAGES % 2 == 0, "slot parity = buffer parity");
  int g = 0;
  for (; g + F6_STAGES <= G; g += F6_STAGES) static_for<0, F6_STAGES>([&](auto j) { group(g + j, j); });
  static_for<0, F6_STAGES - 1>([&](auto j) {
    if (g + j < G) group(g + j, j);
  });
  if ((G - 1) & 1) fold(1);
  else fold(0);
  wait_vmcnt<0>();

  // Epilogue: four tokens of one weight row per lane and block; 16 lanes of a slot write
  // 16 consecutive n of one token.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int mb = m0 + 32 * tg + 16 * i + 4 * slot;
    v4f s4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) s4[t] = mb + t < M ? sa[mb + t] : 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = n0 + 32 * rg + 16 * h + r;
      if (n < N) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (mb + t < M) store_out<BF16>(D, (int64_t)(mb + t) * N + n, acc[h][i][t] * s4[t]);
      }
    }
  }
}

// ---- 128 x 128 tiles, with an optional split of K ------------------------------------
// Per K group a 64 x 128 tile copies 24 KB for 8192 outputs; a 128 x 128 tile 32 KB for
// 16384, so where the copies bound the kernel (a problem with as many 64 x 128 tiles as
// CUs) the wider tile does the same work with a third fewer copies, and a split of K
// keeps all CUs busy.  8 waves in a 4 x 2 grid of 32 x 64 wave tiles: wave w owns tokens
// 32*(w & 3) .. +31 (two FP8 operands) and weight rows 64*(w >> 2) .. +63 (two 32-row
// quarters, four FP6 operands), 8 instructions per K group.  Per stage each wave copies
// 16 activation rows (2 KB); wave w also copies, of weight quarter w & 3, both halves'
// dwords 0-3 (w < 4) or the dwords 4-5 and the quarter's scales (w >= 4).
// SPLIT: the K groups are cut into S slices of GS groups (the last shorter); work item =
// tile * S + slice, and the slice's fp32 partial product (without sa) goes to
// D = P[S][M][N] for launch_scaled_reduce.
constexpr int F7_BM = 128;
constexpr int F7_BN = 128;
constexpr int F7_STAGES = 4;
constexpr int F7_T_OFF = 0;                // activations: 128 rows x 128 B
constexpr int F7_W_OFF = F7_BM * 128;      // weights: 4 quarters x 3072 B
constexpr int F7_S_OFF = F7_W_OFF + 4 * 3072;   // scales: 4 quarters x 1 KB (128 B used)
constexpr int F7_STAGE = F7_S_OFF + 4 * 1024;
constexpr int F7_LOADS = 4;                // copies per wave per stage
static_assert(F7_STAGES * F7_STAGE <= 160 * 1024, "LDS budget");
static_assert((F7_STAGES - 2) * F7_LOADS < 64, "vmcnt range");

template <bool SPLIT, bool BF16>
__global__ void __launch_bounds__(512, 1)
w4a8f6_wide_kernel(int M, int N, int K, int S, int GS, const uint8_t* __restrict__ A,
                   const float* __restrict__ sa, const uint8_t* __restrict__ Bp, const float* __restrict__ Sp,
                   void* __restrict__ D) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F7_STAGES * F7_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tq = wave & 3, rh = wave >> 2;         // token quarter, weight-row half
  const int cq = wave & 3, cr = wave >> 2;         // copy quarter, copy role
  const int r = lane & 15, slot = lane >> 4;

  const int tiles_m = (M + F7_BM - 1) / F7_BM, tiles_n = (N + F7_BN - 1) / F7_BN;
  const int T = tiles_m * tiles_n * (SPLIT ? S : 1);
  int lin = blockIdx.x;
  if ((T & 7) == 0) lin = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int slice = SPLIT ? lin % S : 0;
  if constexpr (SPLIT) lin /= S;
  const int m0 = (lin % tiles_m) * F7_BM, n0 = (lin / tiles_m) * F7_BN;
  const int GA = K / 128;
  const int g0 = SPLIT ? slice * GS : 0;           // this item's groups: g0 .. g0 + G - 1
  const int G = SPLIT ? min(GS, GA - g0) : GA;
  const int G32 = (N + 31) / 32;
  const int64_t Np = 16 * (int64_t)((N + 15) / 16);

  // ---- copy sources (wave-uniform bases plus fixed 32-bit lane offsets; 128 * K < 2^31) ----
  const uint8_t* ua = A + (int64_t)m0 * K + (int64_t)g0 * 128;
  uint32_t va[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (2 * wave + i) + (lane >> 3), u = lane & 7;
    va[i] = (uint32_t)((min(m0 + row, M - 1) - m0) * K + ((u ^ swz8(row)) << 4));
  }
  const uint8_t* ub = Bp + ((int64_t)min(n0 / 32 + cq, G32 - 1) * GA + g0) * 3072 + (cr ? 2048 : 0);
  const uint32_t vb = (uint32_t)lane * 16;
  const int64_t srow0 = min((int64_t)n0 + 32 * cq, Np - 4);
  const uint8_t* us = reinterpret_cast<const uint8_t*>(Sp) + ((int64_t)g0 * Np + srow0) * 4;
  const uint32_t vs = (uint32_t)(min(srow0 + 4 * (lane & 7), Np - 4) - srow0) * 4;
  const uint8_t* u2 = cr ? us : ub + 1024;
  const int64_t step2 = cr ? Np * 4 : 3072;
  const uint32_t v2 = cr ? vs : vb;
  const int w1 = F7_W_OFF + cq * 3072 + (cr ? 2048 : 0);
  const int w2 = cr ? F7_S_OFF + cq * 1024 : w1 + 1024;

  auto issue = [&](int g, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    const int gc = min(g, G - 1);                  // past the end: re-read the last group
    uint8_t* base = smem + SLOT * F7_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_copy16(ua + (int64_t)gc * 128 + va[i], (lds_void*)(base + F7_T_OFF + (2 * wave + i) * 1024));
    lds_copy16(ub + (int64_t)gc * 3072 + vb, (lds_void*)(base + w1));
    lds_copy16(u2 + (int64_t)gc * step2 + v2, (lds_void*)(base + w2));
  };

  // acc[q][h][i]: weight quarter 2rh + q, half h (16 rows), token block i (16 tokens);
  // lane (slot, r) element t holds token 32tq + 16i + 4slot + t and weight row
  // 64rh + 32q + 16h + r.
  v4f acc[2][2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[q][h][i] = v4f{0.f, 0.f, 0.f, 0.f};
  const int unit = 0x7F7F7F7F;

  static_for<0, F7_STAGES - 1>([&](auto p) { issue(p, p); });

  struct Frag { v8i w[2][2]; float s[2][2]; v8i a[2]; };
  Frag fr[2];
  v4f part[2][2][2][2];
  float sc[2][2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[1][q][h] = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) part[1][q][h][i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  auto load = [&](auto slot_c, auto set_c) {
    constexpr int SLOT = decltype(slot_c)::value, SET = decltype(set_c)::value;
    const uint8_t* base = smem + SLOT * F7_STAGE;
    Frag& f = fr[SET];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int quarter = 2 * rh + q;
      const uint8_t* wb = base + F7_W_OFF + quarter * 3072 + lane * 16;
      const v4i w0 = *reinterpret_cast<const v4i*>(wb);
      const v4i w1v = *reinterpret_cast<const v4i*>(wb + 1024);
      const v4i wh = *reinterpret_cast<const v4i*>(wb + 2048);
      f.w[q][0] = v8i{w0[0], w0[1], w0[2], w0[3], wh[0], wh[1], 0, 0};
      f.w[q][1] = v8i{w1v[0], w1v[1], w1v[2], w1v[3], wh[2], wh[3], 0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.s[q][h] = *reinterpret_cast<const float*>(base + F7_S_OFF + quarter * 1024 + (16 * h + r) * 4);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * tq + 16 * i + r;
      const v4i a0 = *reinterpret_cast<const v4i*>(base + F7_T_OFF + row * 128 + (((2 * slot) ^ swz8(row)) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(base + F7_T_OFF + row * 128 + (((2 * slot + 1) ^ swz8(row)) << 4));
      f.a[i] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  };
  auto fold = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[q][h][i][t] = __builtin_fmaf(part[buf][q][h][i][t], sc[buf][q][h], acc[q][h][i][t]);
  };

  auto group = [&](int g, auto j_c) {
    constexpr int J = decltype(j_c)::value, BUF = J & 1;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(F7_STAGES - 3) * F7_LOADS>();
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    issue(g + F7_STAGES - 1, std::integral_constant<int, (J + F7_STAGES - 1) % F7_STAGES>{});
    load(std::integral_constant<int, (J + 1) % F7_STAGES>{}, std::integral_constant<int, BUF ^ 1>{});
    const Frag& f = fr[BUF];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[BUF][q][h] = f.s[q][h];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          part[BUF][q][h][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              f.a[i], f.w[q][h], v4f{0.f, 0.f, 0.f, 0.f}, kFmtFp8, kFmtE3M2, 0, unit, 0, unit);
    fold(BUF ^ 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // a global -> LDS copy
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // five VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  wait_vmcnt<(F7_STAGES - 2) * F7_LOADS>();
  barrier_lds();
  load(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  static_assert(F7_STAGES % 2 == 0, "slot parity = buffer parity");
  int g = 0;
  for (; g + F7_STAGES <= G; g += F7_STAGES) static_for<0, F7_STAGES>([&](auto j) { group(g + j, j); });
  static_for<0, F7_STAGES - 1>([&](auto j) {
    if (g + j < G) group(g + j, j);
  });
  if ((G - 1) & 1) fold(1);
  else fold(0);
  wait_vmcnt<0>();

  if constexpr (SPLIT) D = static_cast<float*>(D) + (int64_t)slice * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int mb = m0 + 32 * tq + 16 * i + 4 * slot;
    v4f s4 = v4f{1.f, 1.f, 1.f, 1.f};
    if constexpr (!SPLIT) {
#pragma unroll
      for (int t = 0; t < 4; ++t) s4[t] = mb + t < M ? sa[mb + t] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + 64 * rh + 32 * q + 16 * h + r;
        if (n < N) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (mb + t < M) store_out<SPLIT ? false : BF16>(D, (int64_t)(mb + t) * N + n, acc[q][h][i][t] * s4[t]);
        }
      }
  }
}

}  // namespace

void w4a8_prepack_fp6_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes) {
  const int64_t G32 = ceil_div(N, 32), G16 = ceil_div(N, 16), G = K / 128;
  *weight_bytes = G32 * G * 3072;
  *scale_bytes = G * 16 * G16 * 4;
}

hipError_t launch_w4a8_prepack_fp6(int64_t N, int64_t K, const uint8_t* B, const uint16_t* sB, uint8_t* Bp6,
                                   float* Sp, hipStream_t s) {
  const int64_t G32 = ceil_div(N, 32), G = K / 128;
  const int64_t cap = device_cus() * 8;
  const int64_t wu = G32 * G * 64;
  const unsigned gw = (unsigned)(ceil_div(wu, 256) < cap ? ceil_div(wu, 256) : cap);
  hipLaunchKernelGGL(w4a8_prepack_fp6_kernel, dim3(gw), dim3(256), 0, s, wu, (int)N, (int)G, K / 2, B, Bp6);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_w4a8_prepack_scales(N, K, sB, Sp, s);
}

bool w4a8_fp6_fits(int64_t K) { return K <= kFp6MaxK; }

// Groups per K slice for `splits` slices of G groups (at least 2).
int fp6_slice_groups(int64_t G, int64_t splits) {
  const int64_t gs = ceil_div(G, splits);
  return (int)(gs < 2 ? 2 : gs);
}

int64_t w4a8_fp6_splits(int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap) {
  const int64_t G = K / 128;
  if (M <= 0 || N <= 0 || G < 4) return 1;
  int64_t S;
  if (requested > 0) {
    S = requested;
  } else {
    // Split only when even the unsplit kernel's 64 x 128 tiles leave CUs idle (at one
    // tile per CU the split's reduction costs what its wider tiles save); then enough
    // slices of 128 x 128 tiles to give every CU an item, each slice at least 8 K groups.
    const int64_t cus = device_cus();
    if (ceil_div(M, F6_BM) * ceil_div(N, F6_BN) >= cus) return 1;
    const int64_t tiles = ceil_div(M, F7_BM) * ceil_div(N, F7_BN);
    S = ceil_div(cus, tiles);
    if (S > G / 8) S = G / 8;
  }
  if (S > kMaxSplits) S = kMaxSplits;
  if (S > cap) S = cap;
  if (S < 2) return 1;
  return ceil_div(G, fp6_slice_groups(G, S));         // the slices that exist
}

hipError_t launch_w4a8_gemm_prepacked_fp6_split(const W4A8Args& a, const float* Sp, int64_t splits, float* P,
                                                hipStream_t s) {
  if (a.K % 128 != 0 || a.K == 0 || a.M <= 0 || a.N <= 0 || !w4a8_fp6_fits(a.K)) return hipErrorInvalidValue;
  if (splits <= 1) return launch_w4a8_gemm_prepacked_fp6(a, Sp, s);
  const int64_t G = a.K / 128;
  const int GS = fp6_slice_groups(G, splits);
  const int64_t S = ceil_div(G, GS);
  if (S > splits || S < 2) return hipErrorInvalidValue;
  const int64_t items = ceil_div(a.M, F7_BM) * ceil_div(a.N, F7_BN) * S;
  if (items > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((w4a8f6_wide_kernel<true, false>), dim3((unsigned)items), dim3(512), 0, s, (int)a.M, (int)a.N,
                     (int)a.K, (int)S, GS, a.A, a.sa, a.B, Sp, static_cast<void*>(P));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_scaled_reduce(1, a.M, a.N, (int)S, P, a.sa, 1.0f, 0, a.D, a.bf16_out, s);
}

hipError_t launch_w4a8_gemm_prepacked_fp6(const W4A8Args& a, const float* Sp, hipStream_t s) {
  if (a.K % 128 != 0 || a.K == 0 || a.M <= 0 || a.N <= 0 || !w4a8_fp6_fits(a.K)) return hipErrorInvalidValue;
  // 64 x 128 tiles while they all run at once (one per CU); beyond that 128 x 128 tiles,
  // which copy a third fewer bytes per output (N = K = 8192, cold weights: M = 384, 512,
  // 1024, 2048 take 44, 44, 88, 173 us against 58, 56, 114, 226 us).
  const int64_t wide = ceil_div(a.M, F7_BM) * ceil_div(a.N, F7_BN);
  if (ceil_div(a.M, F6_BM) * ceil_div(a.N, F6_BN) > device_cus() && wide <= INT32_MAX) {
    if (a.bf16_out)
      hipLaunchKernelGGL((w4a8f6_wide_kernel<false, true>), dim3((unsigned)wide), dim3(512), 0, s, (int)a.M, (int)a.N,
                         (int)a.K, 1, (int)(a.K / 128), a.A, a.sa, a.B, Sp, a.D);
    else
      hipLaunchKernelGGL((w4a8f6_wide_kernel<false, false>), dim3((unsigned)wide), dim3(512), 0, s, (int)a.M,
                         (int)a.N, (int)a.K, 1, (int)(a.K / 128), a.A, a.sa, a.B, Sp, a.D);
    return hipGetLastError();
  }
  const int64_t tiles = ceil_div(a.M, F6_BM) * ceil_div(a.N, F6_BN);
  if (tiles > INT32_MAX) return hipErrorInvalidConfiguration;
  if (a.bf16_out)
    hipLaunchKernelGGL((w4a8f6_gemm_kernel<true>), dim3((unsigned)tiles), dim3(512), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sa, a.B, Sp, a.D);
  else
    hipLaunchKernelGGL((w4a8f6_gemm_kernel<false>), dim3((unsigned)tiles), dim3(512), 0, s, (int)a.M, (int)a.N,
                       (int)a.K, a.A, a.sa, a.B, Sp, a.D);
  return hipGetLastError();
}

}  // namespace fp4g
