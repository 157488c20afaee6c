// MXFP4 GEMM for gfx950: D[M][N] = sum_k e2m1(A[m,k]) 2^(sfA[m,k/32]-127) * e2m1(B[n,k]) 2^(sfB[n,k/32]-127)
//
// The block-scaled product with E8M0 scales per 32 K elements is the one of
// section 1 ("Block-Scaled MXFP4 GEMM in cute-rs (SM120a)") of the cuda-oxide
// page "TMA Pipelines, Tensor Cores, and ctm-rs Interop": packed FP4 K stages
// are consumed as K=64 MMA steps, one E8M0 scale pair per step, fed by a ring of
// asynchronous copies.  The loop nest (output tiles over the grid, a runtime
// K-tile loop, an unrolled inner loop over instructions) follows the tiled-GEMM
// nest of the Hopper CUTLASS/CuTe DSL post, section "Where each level sits in the
// GEMM loop nest"; accumulators start at zero and D is never read (same section,
// the zero-fill form).  The ring depth follows the rule of that post's section
// "The six choices of the SS builder" (choice 5): as many stages as fit on chip.
//
// gfx950 design:
//   * one workgroup of 4 waves per BM x BN output tile, each wave owning a
//     WM x WN sub-tile (128 x 128 at the large configuration: 16 32x32 blocks,
//     256 fp32 accumulators per lane, held in AGPRs);
//   * a K stage is BK elements (BK/2 bytes of packed FP4 per row): 256 when K
//     allows, so every row segment a copy fetches is a whole 128-byte cache line
//     (64-byte half lines cost twice the L1 traffic); 128 otherwise;
//   * the A/B tiles of a stage and their E8M0 scale dwords are copied HBM -> LDS
//     by global_load_lds_dwordx4 / _dword (no VGPR round trip) into a ring of
//     STAGES slots; each wave waits for its own copies with s_waitcnt vmcnt and
//     one s_barrier per stage publishes them;
//   * LDS rows are BK/2 bytes; 16-byte chunk c of row r sits at chunk position
//     c ^ swz(r), so the 8 (or 16) lanes that read one logical chunk of
//     consecutive rows hit distinct banks with ds_read_b128.  A copy instruction
//     writes 1 KB contiguously (lane i -> bytes 16i..16i+15), so lane i fetches
//     the global chunk that belongs at that position;
//   * v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: a stage is NQ = BK/64
//     MFMA quarters; lane l (slot h = l/32) owns chunks NQ*h .. NQ*h+NQ-1 of its
//     row, and quarter kq uses chunk NQ*h+kq with op_sel = kq on the scale dword
//     that holds blocks NQ*h .. NQ*h+3 (shifted when NQ = 2), so every lane's
//     scale byte matches its 32 elements;
//   * inside a stage the fragments of the next quarter are read while the 16
//     MFMAs of the current one run; the barrier sits before the last quarter,
//     whose MFMAs hide the copies for stage s+STAGES (into the slot stage s just
//     released) and the reads of stage s+1's first quarter and scales;
//   * output tiles are numbered so that the tiles resident at once on one XCD
//     (workgroups are dealt round-robin over the 8 XCDs) share A and B panels
//     in that XCD's L2.
//
// Batch and K split.  The problem shape is (M, N, K, L) with L a batch count, all
// runtime values (the Hopper post, section "How a kernel is assembled"); the L
// problems sit back to back in memory and share one persistent grid.  When the
// output tiles cannot fill the CUs (skinny or small problems: the post's
// introduction names a stream-K scheduler as the load-balancing variant of the
// persistent one), the K loop of every tile is cut into S slices that run as
// separate work items and write fp32 partial sums; a second kernel adds the S
// partials of each element in slice order and converts.  No workgroup waits on
// another, and the sum order is fixed, so results are reproducible bit for bit.
#include <type_traits>

#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

// Chunk swizzles: rows of 4 chunks (64 B) and of 8 chunks (128 B).  Consecutive
// rows read at one logical chunk land in distinct 16-byte bank groups within any
// 8 (mod 128 B) or 16 (mod 256 B) lane group.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
template <int CHUNKS>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CHUNKS == 4) return swz4(r);
  else return swz8(r);
}

// One work item: output tile (tm, tn) of problem b of the batch, K slice s.
struct Item { int b, s, tm, tn; };

// Map a linear work id to an item.  Consecutive ids are dealt to the 8 XCDs in turn;
// they are regrouped so each XCD owns a contiguous range of the item order, in which
// the K slices of one tile are adjacent and the tiles of one problem follow a grouped
// (G tile rows at a time) order, so the tiles resident at once on an XCD share A and
// B panels in its L2.
__device__ __forceinline__ Item item_of(int wg, int total, int S, int tiles_m, int tiles_n) {
  int lin = wg;
  if ((total & 7) == 0) lin = (wg & 7) * (total >> 3) + (wg >> 3);
  Item it;
  const int T = tiles_m * tiles_n;
  it.s = lin % S;
  const int r = lin / S;
  it.b = r / T;
  const int t = r - it.b * T;
  constexpr int G = 8;
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gsize = min(G, tiles_m - first_m);
  const int in_group = t - group * G * tiles_n;
  it.tm = first_m + in_group % gsize;
  it.tn = in_group / gsize;
  return it;
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES>
struct Cfg {
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = BK / 2;              // bytes of one row per stage
  static constexpr int CHUNKS = ROWB / 16;         // 16-byte chunks per row
  static constexpr int NQ = BK / 64;               // MFMA quarters per stage
  static constexpr int SDW = BK / 128;             // scale dwords per row per stage
  static constexpr int RPC = 1024 / ROWB;          // rows per 1 KB copy
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;            // scales: [SDW][rows] dwords
  static constexpr int SB_OFF = SA_OFF + SDW * BM * 4;
  static constexpr int STAGE = SB_OFF + SDW * BN * 4;
  static constexpr int LDS = STAGE * STAGES;
  static constexpr int IA = BM / RPC / NW, IB = BN / RPC / NW;   // 1 KB copies per wave per stage
  static constexpr int TSA = SDW * BM / 64, TSB = SDW * BN / 64;  // 256 B scale copies per stage
  static constexpr int SCA = (TSA + NW - 1) / NW, SCB = (TSB + NW - 1) / NW;   // per wave
  static constexpr int LOADS = IA + IB + SCA + SCB;             // copies per wave per stage
  static_assert(BK == 128 || BK == 256, "stage size");
  static_assert(IA >= 1 && IB >= 1 && BM % (RPC * NW) == 0 && BN % (RPC * NW) == 0, "tile/waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies cover 64 rows");
  static_assert(STAGE % 256 == 0, "stage alignment");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && (STAGES - 1) * LOADS < 64, "vmcnt range");
};

// L problems of one shape stored back to back: A [L][M][K/2], sfA [L][M][K/32], B
// [L][N][K/2], sfB [L][N][K/32].  Without SPLIT, D is [L][M][N] of the output type.
// With SPLIT, the K stages are cut into S slices of (near) equal length, every
// (problem, tile, slice) is one work item, and D is the fp32 partial-sum buffer
// [L][S][M][N] that splitk_reduce_kernel folds into the output.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool BF16, bool SPLIT>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
mxfp4_gemm_kernel(int M, int N, int K, int L, int S, const uint8_t* __restrict__ A,
                  const uint8_t* __restrict__ sfA, const uint8_t* __restrict__ B,
                  const uint8_t* __restrict__ sfB, void* __restrict__ D) {
  using C = Cfg<BM, BN, WM, WN, BK, STAGES>;
  constexpr int NWN = BN / WN;
  constexpr int FI = WM / 32, FJ = WN / 32;
  constexpr int NQ = C::NQ;

  // Output panels.  The epilogue stages the wave tile through LDS in panels of PB bytes
  // per row.  With 256 x 256 tiles (one workgroup per CU) the panels sit past the ring,
  // in the LDS the ring leaves free, so the next tile's first copies can land while
  // this tile's output is written; otherwise they reuse the ring.
  constexpr bool OUT_BF16 = BF16 && !SPLIT;
  constexpr int ELEM = OUT_BF16 ? 2 : 4;
  constexpr bool EPI_SPARE = BM == 256 && BN == 256;
  constexpr int EPI_AVAIL = EPI_SPARE ? 160 * 1024 - C::LDS : C::LDS;
  constexpr int PR = EPI_SPARE ? 32 : WM;                   // panel rows
  constexpr int PFIT = EPI_AVAIL / (C::NW * PR) - 16;
  constexpr int PB0 = (WN * ELEM < 256) ? WN * ELEM : 256;
  constexpr int PB = PB0 <= PFIT ? PB0 : PB0 / 2 <= PFIT ? PB0 / 2 : PB0 / 4;   // panel bytes per row
  constexpr int PW = PB / ELEM;                             // panel columns
  constexpr int RS = PB + 16;                               // LDS row stride
  constexpr int LPR = PB / 16, RPI = 64 / LPR;              // lanes per row, rows per read
  static_assert(PB >= 8 * ELEM && WN % PW == 0 && PW % 8 == 0, "panels hold whole 8-column groups");
  static_assert(C::NW * PR * RS <= EPI_AVAIL && PR % RPI == 0, "output panels fit");
  constexpr int EPI_OFF = EPI_SPARE ? C::LDS : 0;
  constexpr int SMEM = EPI_SPARE ? C::LDS + C::NW * PR * RS : C::LDS;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int hi = lane >> 5, r32 = lane & 31;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = L * tiles_m * tiles_n * S;
  // Persistent: the grid is at most one workgroup per CU and each workgroup walks its
  // work items.  A tile's output stores drain while the next tile's copies and MFMAs
  // run, instead of every CU writing its tile at the same moment.
  if ((int)blockIdx.x >= total) return;
  const int64_t lda = K / 2, ldsf = K / 32;
  const int KT = K / BK;

  // The current work item: its tile, its K stages ks0 .. ks0+KS-1 of the KT stages
  // (KS >= 1: S <= KT), and this lane's copy sources.
  Item it;
  int m0 = 0, n0 = 0, KS = 1;
  const uint8_t* ga[C::IA];
  const uint8_t* gb[C::IB];
  const uint8_t* gsa[C::SCA];
  const uint8_t* gsb[C::SCB];
  int lsa[C::SCA], lsb[C::SCB];
  auto setup = [&](int work) {
    it = item_of(work, total, S, tiles_m, tiles_n);
    m0 = it.tm * BM;
    n0 = it.tn * BN;
    const int ks0 = (int)((int64_t)it.s * KT / S);
    KS = (int)((int64_t)(it.s + 1) * KT / S) - ks0;
    const uint8_t* Ab = A + (int64_t)it.b * M * lda + (int64_t)ks0 * C::ROWB;
    const uint8_t* Bb = B + (int64_t)it.b * N * lda + (int64_t)ks0 * C::ROWB;
    const uint8_t* sfAb = sfA + (int64_t)it.b * M * ldsf + (int64_t)ks0 * 4 * C::SDW;
    const uint8_t* sfBb = sfB + (int64_t)it.b * N * ldsf + (int64_t)ks0 * 4 * C::SDW;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) {
      const int row = C::RPC * (wave * C::IA + i) + lane / C::CHUNKS;
      const int c = (lane % C::CHUNKS) ^ swz<C::CHUNKS>(row);
      ga[i] = Ab + (int64_t)min(m0 + row, M - 1) * lda + c * 16;
    }
#pragma unroll
    for (int i = 0; i < C::IB; ++i) {
      const int row = C::RPC * (wave * C::IB + i) + lane / C::CHUNKS;
      const int c = (lane % C::CHUNKS) ^ swz<C::CHUNKS>(row);
      gb[i] = Bb + (int64_t)min(n0 + row, N - 1) * lda + c * 16;
    }
    // Scale copy z covers dword d = z / (rows/64) of 64 rows (block z % (rows/64)).  When
    // there are fewer copies than waves, waves repeat one (identical bytes, same place).
#pragma unroll
    for (int j = 0; j < C::SCA; ++j) {
      const int z = (wave * C::SCA + j) % C::TSA, d = z / (BM / 64), blk = z % (BM / 64);
      gsa[j] = sfAb + (int64_t)min(m0 + 64 * blk + lane, M - 1) * ldsf + 4 * d;
      lsa[j] = C::SA_OFF + d * BM * 4 + 256 * blk;
    }
#pragma unroll
    for (int j = 0; j < C::SCB; ++j) {
      const int z = (wave * C::SCB + j) % C::TSB, d = z / (BN / 64), blk = z % (BN / 64);
      gsb[j] = sfBb + (int64_t)min(n0 + 64 * blk + lane, N - 1) * ldsf + 4 * d;
      lsb[j] = C::SB_OFF + d * BN * 4 + 256 * blk;
    }
  };

  // Copy q (0 .. LOADS-1) of stage ks into ring slot ks % STAGES: A chunks, B chunks,
  // then the scale blocks.  Stages past the end re-read the last stage (the copies land
  // in slots nobody reads), which keeps the loop branch-free.
  auto issue_one = [&](int ks, int q) {
    const int st = ks % STAGES;
    const int kc = min(ks, KS - 1);
    uint8_t* base = smem + st * C::STAGE;
    const int64_t kb = (int64_t)kc * C::ROWB;
    if (q < C::IA) {
      lds_copy16(ga[q] + kb, (lds_void*)(base + 1024 * (wave * C::IA + q)));
    } else if (q < C::IA + C::IB) {
      const int i = q - C::IA;
      lds_copy16(gb[i] + kb, (lds_void*)(base + C::A_BYTES + 1024 * (wave * C::IB + i)));
    } else if (q < C::IA + C::IB + C::SCA) {
      const int j = q - C::IA - C::IB;
      lds_copy4(gsa[j] + kc * 4 * C::SDW, (lds_void*)(base + lsa[j]));
    } else {
      const int j = q - C::IA - C::IB - C::SCA;
      lds_copy4(gsb[j] + kc * 4 * C::SDW, (lds_void*)(base + lsb[j]));
    }
  };
  auto issue = [&](int ks) {
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q) issue_one(ks, q);
  };

  // ---- LDS read offsets of this lane's fragments ----
  int ra[FI], rb[FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i) ra[i] = wm * WM + i * 32 + r32;
#pragma unroll
  for (int j = 0; j < FJ; ++j) rb[j] = wn * WN + j * 32 + r32;

  v4i fa[2][FI], fb[2][FJ];
  int sa[FI], sb[FJ];     // scales of the stage being computed
  int na[FI], nb[FJ];     // scales of the next stage, read during the current one
  // Fragment r (0 .. FI+FJ-1: A blocks, then B blocks) of quarter kq of stage ks.
  auto read_frag = [&](int ks, int kq, int set, int r) {
    const uint8_t* base = smem + (ks % STAGES) * C::STAGE;
    const int c = NQ * hi + kq;
    if (r < FI)
      fa[set][r] = *reinterpret_cast<const v4i*>(base + ra[r] * C::ROWB + ((c ^ swz<C::CHUNKS>(ra[r])) << 4));
    else
      fb[set][r - FI] = *reinterpret_cast<const v4i*>(base + C::A_BYTES + rb[r - FI] * C::ROWB +
                                                      ((c ^ swz<C::CHUNKS>(rb[r - FI])) << 4));
  };
  auto read_frags = [&](int ks, int kq, int set) {
#pragma unroll
    for (int r = 0; r < FI + FJ; ++r) read_frag(ks, kq, set, r);
  };
  // Scale dword r (A blocks, then B blocks) of stage ks into the next-stage set: the dword
  // holding blocks NQ*hi .., shifted so op_sel = kq picks block NQ*hi + kq.
  auto read_scale = [&](int ks, int r) {
    const uint8_t* base = smem + (ks % STAGES) * C::STAGE;
    const int d = (NQ * hi) >> 2, sh = 8 * ((NQ * hi) & 3);
    if (r < FI)
      na[r] = (int)(*reinterpret_cast<const uint32_t*>(base + C::SA_OFF + d * BM * 4 + 4 * ra[r]) >> sh);
    else
      nb[r - FI] = (int)(*reinterpret_cast<const uint32_t*>(base + C::SB_OFF + d * BN * 4 + 4 * rb[r - FI]) >> sh);
  };
  auto read_scales = [&](int ks) {
#pragma unroll
    for (int r = 0; r < FI + FJ; ++r) read_scale(ks, r);
  };
  auto take_scales = [&]() {
#pragma unroll
    for (int i = 0; i < FI; ++i) sa[i] = na[i];
#pragma unroll
    for (int j = 0; j < FJ; ++j) sb[j] = nb[j];
  };

  v16f acc[FI][FJ];

  // The MFMAs of quarter KQ (register set SET); after MFMA q, `extra(q)` issues that
  // slot's memory instructions, in a fixed order (sched_barrier pins it), so their issue
  // hides under the MFMA pipe.
  auto quarter = [&](auto kq_c, auto set_c, auto&& extra) {
    constexpr int KQ = decltype(kq_c)::value, SET = decltype(set_c)::value;
#pragma unroll
    for (int q = 0; q < FI * FJ; ++q) {
      const int i = q / FJ, j = q % FJ;
      // B first: the accumulator holds D^T, so a lane owns 4 consecutive columns of a row
      acc[i][j] = mfma_fp4_32x32<KQ>(fb[SET][j], fa[SET][i], acc[i][j], sb[j], sa[i]);
      __builtin_amdgcn_sched_barrier(0);
      extra(q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The copies of stage j are issued in two halves: copies 0 .. LH-1 under the last
  // quarter of stage j-STAGES (right after the barrier that frees its slot), copies
  // LH .. LOADS-1 under the first quarter of stage j-STAGES+1.
  constexpr int LH = (C::LOADS + 1) / 2;
  // Quarter KQ (not the last) while reading quarter KQ+1's fragments into the other set;
  // quarter 0 also issues the second half of stage ks+STAGES-1's copies.
  auto mid_quarter = [&](int ks, auto kq_c) {
    constexpr int KQ = decltype(kq_c)::value;
    quarter(kq_c, std::integral_constant<int, (KQ & 1)>{}, [&](int q) {
      if (q < FI + FJ) read_frag(ks, KQ + 1, (KQ + 1) & 1, q);
      __builtin_amdgcn_sched_barrier(0);
      if (KQ == 0 && q < C::LOADS - LH) issue_one(ks + STAGES - 1, LH + q);
    });
#pragma unroll
    for (int q = FI * FJ; q < FI + FJ; ++q) read_frag(ks, KQ + 1, (KQ + 1) & 1, q);
    if constexpr (KQ == 0) {
#pragma unroll
      for (int q = FI * FJ; q < C::LOADS - LH; ++q) issue_one(ks + STAGES - 1, LH + q);
    }
  };

  // ---- prologue copies of the current item: stages 0 .. STAGES-2 and the first half
  // of stage STAGES-1 ----
  auto prologue = [&]() {
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(p);
#pragma unroll
    for (int q = 0; q < LH; ++q) issue_one(STAGES - 1, q);
  };

  int work = blockIdx.x;
  setup(work);
  prologue();
  while (true) {
  // Stage 0 has landed once at most the first half of stage STAGES-1 (and the STAGES-2
  // stages before it) is in flight.  Output stores of the previous tile issued after
  // these copies only make the wait longer: copies complete in order, so while any
  // copy of stage 0 is pending, every later copy is too.
  wait_vmcnt<(STAGES - 2) * C::LOADS + LH>();
  barrier_lds();
  read_scales(0);
  take_scales();
  read_frags(0, 0, 0);
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v16f{};

  // One stage per iteration, no branches in the body (so the compiler keeps the order):
  //   quarters 0 .. NQ-2: MFMAs of quarter kq, reading quarter kq+1's fragments;
  //   this wave's copies of stage ks+1 complete; the barrier publishes everyone's and
  //     certifies that every wave has finished reading slot ks % STAGES;
  //   quarter NQ-1: MFMAs, while issuing the copies of stage ks+STAGES into that slot
  //     and reading stage ks+1's first-quarter fragments and scales;
  //   the next scales become current.
  // On the last stages the reads of stage ks+1 hit a slot holding a re-read copy; the
  // values are unused.
  constexpr int LQ = NQ - 1;
  static_assert((LQ & 1) == 1, "the last quarter uses register set 1");
  for (int ks = 0; ks < KS; ++ks) {
    mid_quarter(ks, std::integral_constant<int, 0>{});
    if constexpr (NQ == 4) {
      mid_quarter(ks, std::integral_constant<int, 1>{});
      mid_quarter(ks, std::integral_constant<int, 2>{});
    }
    // Stage ks+1's copies are complete once at most the STAGES-2 stages issued after them
    // (ks+2 .. ks+STAGES-1, both halves) are in flight.
    wait_vmcnt<(STAGES - 2) * C::LOADS>();
    barrier_lds();
    quarter(std::integral_constant<int, LQ>{}, std::integral_constant<int, 1>{}, [&](int q) {
      if (q < LH) issue_one(ks + STAGES, q);
      __builtin_amdgcn_sched_barrier(0);
      if (q < FI + FJ) read_frag(ks + 1, 0, 0, q);
      __builtin_amdgcn_sched_barrier(0);
      if (q < FI + FJ) read_scale(ks + 1, q);
    });
#pragma unroll
    for (int q = FI * FJ; q < LH; ++q) issue_one(ks + STAGES, q);
#pragma unroll
    for (int q = FI * FJ; q < FI + FJ; ++q) {
      read_frag(ks + 1, 0, 0, q);
      read_scale(ks + 1, q);
    }
    take_scales();
  }
  // No copy may still be landing in LDS when the ring is reused or the workgroup exits.
  wait_vmcnt<0>();
  // Every wave's copies have landed and nobody reads the ring any more: its LDS is free.
  barrier_lds();

  // The output coordinates of this item; with the panels past the ring, the next item's
  // first copies go out now and land while this tile's output is written.
  const int eb = it.b, es = it.s, em0 = m0, en0 = n0;
  const int next = work + (int)gridDim.x;
  if constexpr (EPI_SPARE) {
    if (next < total) {
      setup(next);
      prologue();
    }
  }

  // Epilogue.  The accumulator of block (i, j) is D^T: lane (hi, r32) holds row
  // m = i*32 + r32 of the wave tile and, for g = 0..3, the four consecutive columns
  // j*32 + 8g + 4hi + 0..3.  When D's rows are whole 16-byte units the wave tile goes
  // through its own LDS region (rows padded to PB+16 bytes) in panels of PR rows x PW
  // columns, and is read back row-wise so each lane stores 16 contiguous bytes and a store
  // instruction writes 64/(PB/16) whole row segments.  Otherwise each group of four
  // goes out directly.
  uint8_t* const Dt = static_cast<uint8_t*>(D) + (SPLIT ? (int64_t)eb * S + es : (int64_t)eb) * M * N * ELEM;
  const int mw = em0 + wm * WM, nw = en0 + wn * WN;
  if ((N % (16 / ELEM)) == 0) {
    uint8_t* region = smem + EPI_OFF + wave * (PR * RS);
#pragma unroll
    for (int ib = 0; ib < WM / PR; ++ib)
#pragma unroll
    for (int p = 0; p < WN / PW; ++p) {
#pragma unroll
      for (int ii = 0; ii < PR / 32; ++ii)
#pragma unroll
        for (int c8 = 0; c8 < PW / 8; ++c8) {
          const int i = ib * (PR / 32) + ii;
          const int col = p * PW + 8 * c8;              // first column of the 8-column group
          const int j = col / 32, g = (col % 32) / 8;
          uint8_t* dst = region + (ii * 32 + r32) * RS + (8 * c8 + 4 * hi) * ELEM;
          const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if constexpr (OUT_BF16) {
            typedef unsigned int v2u __attribute__((ext_vector_type(2)));
            *reinterpret_cast<v2u*>(dst) = v2u{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          } else {
            *reinterpret_cast<v4f*>(dst) = v4f{v0, v1, v2, v3};
          }
        }
#pragma unroll
      for (int rd = 0; rd < PR / RPI; ++rd) {
        const int r = rd * RPI + lane / LPR, ch = lane % LPR;
        const v4i val = *reinterpret_cast<const v4i*>(region + r * RS + ch * 16);
        const int m = mw + ib * PR + r, n = nw + p * PW + ch * (16 / ELEM);
        if (m < M && n < N)
          *reinterpret_cast<v4i*>(Dt + ((int64_t)m * N + n) * ELEM) = val;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int m = mw + i * 32 + r32;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nw + j * 32 + 8 * g + 4 * hi;
          const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if (m < M) store_out4<OUT_BF16>(Dt, (int64_t)m * N + n, N - n, v0, v1, v2, v3);
        }
      }
    }
  }
  if constexpr (!EPI_SPARE) {
    // No wave may start the next tile's copies into LDS while another still reads its
    // output panel.
    barrier_lds();
    if (next < total) {
      setup(next);
      prologue();
    }
  }
  if (next >= total) break;
  work = next;
  }  // work-item loop
}

// D[b][i] = sum over s = 0, 1, .., S-1 (in that order) of P[b][s][i], i < MN, converted
// to the output type.  VEC: four consecutive elements per lane (MN % 4 == 0).
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(int64_t MN, int L, int S, const float* __restrict__ P, void* __restrict__ D) {
  constexpr int W = VEC ? 4 : 1;
  const int64_t per = MN / W, total = per * L;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (int64_t)gridDim.x * 256) {
    const int64_t b = u / per, i = (u - b * per) * W;
    const float* p = P + b * S * MN + i;
    if constexpr (VEC) {
      v4f acc = *reinterpret_cast<const v4f*>(p);
      for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const v4f*>(p + s * MN);
      store_out4<BF16>(D, b * MN + i, 4, acc[0], acc[1], acc[2], acc[3]);
    } else {
      float acc = p[0];
      for (int s = 1; s < S; ++s) acc += p[s * MN];
      store_out<BF16>(D, b * MN + i, acc);
    }
  }
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool SPLIT>
hipError_t launch_cfg(const FP4Args& a, int64_t L, int S, void* out, hipStream_t s) {
  using C = Cfg<BM, BN, WM, WN, BK, STAGES>;
  const int64_t items = L * ceil_div(a.M, BM) * ceil_div(a.N, BN) * S;
  if (items > INT32_MAX) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)(items < device_cus() ? items : device_cus());
  if (SPLIT || !a.bf16_out)
    hipLaunchKernelGGL((mxfp4_gemm_kernel<BM, BN, WM, WN, BK, STAGES, false, SPLIT>), dim3(grid), dim3(C::NT),
                       0, s, (int)a.M, (int)a.N, (int)a.K, (int)L, S, a.A, a.sfA, a.B, a.sfB, out);
  else
    hipLaunchKernelGGL((mxfp4_gemm_kernel<BM, BN, WM, WN, BK, STAGES, true, false>), dim3(grid), dim3(C::NT),
                       0, s, (int)a.M, (int)a.N, (int)a.K, (int)L, S, a.A, a.sfA, a.B, a.sfB, out);
  return hipGetLastError();
}

hipError_t launch_reduce(const FP4Args& a, int64_t L, int S, const float* P, hipStream_t s) {
  const int64_t MN = a.M * a.N;
  const bool vec = MN % 4 == 0;
  const int64_t units = L * (vec ? MN / 4 : MN);
  const int64_t cap = device_cus() * 8;
  const unsigned grid = (unsigned)(ceil_div(units, 256) < cap ? ceil_div(units, 256) : cap);
  if (a.bf16_out) {
    if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<true, true>), dim3(grid), dim3(256), 0, s, MN, (int)L, S, P, a.D);
    else hipLaunchKernelGGL((splitk_reduce_kernel<true, false>), dim3(grid), dim3(256), 0, s, MN, (int)L, S, P, a.D);
  } else {
    if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<false, true>), dim3(grid), dim3(256), 0, s, MN, (int)L, S, P, a.D);
    else hipLaunchKernelGGL((splitk_reduce_kernel<false, false>), dim3(grid), dim3(256), 0, s, MN, (int)L, S, P, a.D);
  }
  return hipGetLastError();
}

// K stages of the 128 x 128 configuration that the split path uses.
int64_t split_stages(int64_t K) { return K % 256 == 0 ? K / 256 : K / 128; }

// One problem of a few tokens runs the decode GEMV instead of the GEMM tiles: 1 to 32
// tokens where fp4_gemv takes them and K >= 4096.  Measured against the GEMM with its
// automatic K split (cold weights, M = 1 ... 32): 7.5-10.0 against 13.6-15.3 us at
// N = 14336, K = 4096; 4.7-6.3 against 9.6-11.1 us at N = K = 4096; 9.1-15.7 against
// 14.5-15.9 us at N = K = 8192; at K = 1024 the GEMM was faster (4.5-5.2 against
// 4.8-7.4 us at N = 2048).
bool decode_route(int64_t L, int64_t M, int64_t K) { return L == 1 && K >= 4096 && fp4_gemv_fits(M, K); }

}  // namespace

int64_t mxfp4_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap) {
  const int64_t KT = split_stages(K);
  int64_t smax = KT < kMaxSplits ? KT : kMaxSplits;
  if (cap < smax) smax = cap;
  if (smax < 2 || L * M * N == 0) return 1;
  if (requested > 0) return requested < smax ? requested : smax;
  if (decode_route(L, M, K)) return 1;
  // Automatic choice.  Problems that already fill the chip with 256 x 256 tiles are not
  // split.  Otherwise model the time of the 128 x 128 path as (rounds of work items over
  // the CUs) x (stages per item + a fixed cost per item) plus the reduction's HBM
  // traffic, and take the cheapest S; one slice needs at least 4 stages.
  const int64_t cus = device_cus();
  if (L * ceil_div(M, 256) * ceil_div(N, 256) >= cus) return 1;
  const int64_t items = L * ceil_div(M, 128) * ceil_div(N, 128);
  const double stage_us = 0.6 * (K % 256 == 0 ? 1.0 : 0.5), item_us = 2.0 * stage_us;
  const double bytes_per_us = 4.0e6;
  int64_t best = 1;
  double best_t = 0;
  for (int64_t S = 1; S <= smax && (S == 1 || KT / S >= 4); ++S) {
    const double rounds = (double)ceil_div(items * S, cus);
    double t = rounds * ((double)KT / S * stage_us + item_us);
    if (S > 1) t += (double)(L * M * N) * 4.0 * (S + 1) / bytes_per_us;
    if (S == 1 || t < best_t) { best = S; best_t = t; }
  }
  return best;
}

hipError_t launch_mxfp4_gemm_batched(const FP4Args& a, int64_t L, int64_t S, float* P, hipStream_t s) {
  if (S <= 1 && decode_route(L, a.M, a.K)) return launch_fp4_gemv(a, s);
  const bool k256 = a.K % 256 == 0;
  if (S > 1) {
    hipError_t e;
    if (a.M <= 64)   // 64-row tiles: no half-empty 128-row tiles (64 x 8192 x 8192: 18.6 -> 17.8 us)
      e = k256 ? launch_cfg<64, 128, 32, 64, 256, 2, true>(a, L, (int)S, P, s)
               : launch_cfg<64, 128, 32, 64, 128, 4, true>(a, L, (int)S, P, s);
    else
      e = k256 ? launch_cfg<128, 128, 64, 64, 256, 2, true>(a, L, (int)S, P, s)
               : launch_cfg<128, 128, 64, 64, 128, 4, true>(a, L, (int)S, P, s);
    if (e != hipSuccess) return e;
    return launch_reduce(a, L, (int)S, P, s);
  }
  const int64_t t256 = L * ceil_div(a.M, 256) * ceil_div(a.N, 256);
  const int64_t t128 = L * ceil_div(a.M, 128) * ceil_div(a.N, 128);
  if (t256 >= 256) {
    if (k256) return launch_cfg<256, 256, 128, 128, 256, 2, false>(a, L, 1, a.D, s);
    return launch_cfg<256, 256, 128, 128, 128, 4, false>(a, L, 1, a.D, s);
  }
  if (t128 >= 128) {
    if (k256) return launch_cfg<128, 128, 64, 64, 256, 2, false>(a, L, 1, a.D, s);
    return launch_cfg<128, 128, 64, 64, 128, 4, false>(a, L, 1, a.D, s);
  }
  return launch_cfg<64, 64, 32, 32, 128, 4, false>(a, L, 1, a.D, s);
}

hipError_t launch_mxfp4_gemm(const FP4Args& a, hipStream_t s) { return launch_mxfp4_gemm_batched(a, 1, 1, nullptr, s); }

}  // namespace fp4g
