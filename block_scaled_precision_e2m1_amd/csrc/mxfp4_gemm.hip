// MXFP4 GEMM for gfx950: D[M][N] = sum_k e2m1(A[m,k]) 2^(sfA[m,k/32]-127) * e2m1(B[n,k]) 2^(sfB[n,k/32]-127)
//
// The block-scaled product with E8M0 scales per 32 K elements is the one of
// section 1 ("Block-Scaled MXFP4 GEMM in cute-rs (SM120a)") of the cuda-oxide
// page "TMA Pipelines, Tensor Cores, and ctm-rs Interop": each 128-element K
// stage of packed FP4 is consumed as two K=64 MMA steps, one E8M0 scale pair
// per step, fed by a multi-stage ring of asynchronous copies.  The loop nest
// (output tiles over the grid, a runtime K-tile loop, an unrolled inner loop
// over instructions) follows the tiled-GEMM nest of the Hopper CUTLASS/CuTe DSL
// post, section "Where each level sits in the GEMM loop nest"; accumulators
// start at zero and D is never read (same section, the zero-fill form).  The
// ring depth follows the rule of that post's section "The six choices of the
// SS builder" (choice 5): as many stages as fit in the on-chip memory.
//
// gfx950 design:
//   * one workgroup of 4 waves per BM x BN output tile, each wave owning a
//     WM x WN sub-tile (128 x 128 at the large configuration: 16 32x32 blocks,
//     256 fp32 accumulators per lane, held in AGPRs);
//   * K advances 128 elements (64 bytes of packed FP4 per row) per step.  The
//     A/B tiles and their E8M0 scale dwords of a step are copied HBM -> LDS by
//     global_load_lds_dwordx4 / _dword (no VGPR round trip) into a STAGES-deep
//     ring, issued STAGES-1 steps ahead; each wave waits for its own copies with
//     s_waitcnt vmcnt and one s_barrier per step publishes them;
//   * LDS rows are 64 bytes; the four 16-byte chunks of row r sit at chunk
//     position c ^ swz(r), so 8 (or 16) lanes reading one logical chunk of
//     consecutive rows hit distinct banks with ds_read_b128.  A copy instruction
//     writes 1 KB contiguously (lane i -> bytes 16i..16i+15), so lane i fetches
//     the global chunk that belongs at that position;
//   * v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: lane l (slot h = l/32)
//     holds chunks 2h and 2h+1 of its row, i.e. K blocks {2h, 2h+1}; the MFMA of
//     half kk uses chunk 2h+kk with op_sel = kk on the row's scale dword shifted
//     right by 16*h, so every lane's scale byte matches its 32 elements;
//   * the fragments of the next half step are read from LDS while the MFMAs of
//     the current one run (two register sets), and the barrier sits between the
//     two halves, so the MFMA pipe is fed across it;
//   * output tiles are numbered so that the tiles resident at once on one XCD
//     (workgroups are dealt round-robin over the 8 XCDs) share A and B panels
//     in that XCD's L2.
#include "common.hpp"
#include "internal.h"

namespace fp4g {
namespace {

constexpr int kBK = 128;            // K elements per step
constexpr int kRowBytes = kBK / 2;  // 64 bytes of packed FP4 per row per step

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

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

// Map a linear workgroup id to an output tile (tm, tn).  Consecutive ids are dealt
// to the 8 XCDs in turn; they are regrouped so each XCD owns a contiguous range of
// a grouped (G tile rows at a time) tile order.
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int T = tiles_m * tiles_n;
  int lin = wg;
  if ((T & 7) == 0) lin = (wg & 7) * (T >> 3) + (wg >> 3);
  constexpr int G = 8;
  const int group = lin / (G * tiles_n);
  const int first_m = group * G;
  const int gsize = min(G, tiles_m - first_m);
  const int in_group = lin - group * G * tiles_n;
  *tm = first_m + in_group % gsize;
  *tn = in_group / gsize;
}

template <int BM, int BN, int WM, int WN, int STAGES>
struct Cfg {
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int NT = NW * 64;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int SA_OFF = A_BYTES + B_BYTES, SB_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = SB_OFF + BN * 4;
  static constexpr int LDS = STAGE * STAGES;
  static constexpr int IA = BM / 16 / NW, IB = BN / 16 / NW;   // 1 KB copies per wave per step
  static constexpr int SCA = BM / 64, SCB = BN / 64;           // 256 B scale copies per step
  static constexpr int LOADS = IA + IB + 2;                    // copies per wave per step
  static_assert(IA >= 1 && IB >= 1 && BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "tile/waves");
  static_assert(SCA >= 1 && SCB >= 1 && NW % SCA == 0 && NW % SCB == 0, "scale copies");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int BM, int BN, int WM, int WN, int STAGES, bool BF16>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
mxfp4_gemm_kernel(int M, int N, int K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ sfA,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ sfB, void* __restrict__ D) {
  using C = Cfg<BM, BN, WM, WN, STAGES>;
  constexpr int NWN = BN / WN;
  constexpr int FI = WM / 32, FJ = WN / 32;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int hi = lane >> 5, r32 = lane & 31;

  int tm, tn;
  tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int64_t lda = K / 2, ldsf = K / 32;
  const int KT = K / kBK;

  // ---- copy sources: this lane's global rows / chunks for each of its copies ----
  const uint8_t* ga[C::IA];
  const uint8_t* gb[C::IB];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) {
    const int row = 16 * (wave * C::IA + i) + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    ga[i] = A + (int64_t)min(m0 + row, M - 1) * lda + c * 16;
  }
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    const int row = 16 * (wave * C::IB + i) + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    gb[i] = B + (int64_t)min(n0 + row, N - 1) * lda + c * 16;
  }
  // scale copies: wave w copies 64 rows of sfA (block w % SCA) and of sfB (block w % SCB);
  // waves beyond the block count repeat a block (identical bytes to identical places).
  const int sca_blk = wave % C::SCA, scb_blk = wave % C::SCB;
  const uint8_t* gsa = sfA + (int64_t)min(m0 + 64 * sca_blk + lane, M - 1) * ldsf;
  const uint8_t* gsb = sfB + (int64_t)min(n0 + 64 * scb_blk + lane, N - 1) * ldsf;

  // Copies of step kt into ring slot kt % STAGES.  Steps past the end re-read the last
  // step (the copies land in slots nobody reads), which keeps the loop branch-free.
  auto issue = [&](int kt) {
    const int st = kt % STAGES;
    const int ks = min(kt, KT - 1);
    uint8_t* base = smem + st * C::STAGE;
    const int64_t kb = (int64_t)ks * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::IA; ++i)
      lds_copy16(ga[i] + kb, (lds_void*)(base + 1024 * (wave * C::IA + i)));
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
      lds_copy16(gb[i] + kb, (lds_void*)(base + C::A_BYTES + 1024 * (wave * C::IB + i)));
    lds_copy4(gsa + ks * 4, (lds_void*)(base + C::SA_OFF + 256 * sca_blk));
    lds_copy4(gsb + ks * 4, (lds_void*)(base + C::SB_OFF + 256 * scb_blk));
  };

  // ---- LDS read offsets of this lane's fragments ----
  int ra[FI], rb[FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i) ra[i] = wm * WM + i * 32 + r32;
#pragma unroll
  for (int j = 0; j < FJ; ++j) rb[j] = wn * WN + j * 32 + r32;

  v4i fa[2][FI], fb[2][FJ];
  int sa[FI], sb[FJ];
  auto read_frags = [&](int kt, int kk, int set) {
    const uint8_t* base = smem + (kt % STAGES) * C::STAGE;
    const int c = 2 * hi + kk;
#pragma unroll
    for (int i = 0; i < FI; ++i)
      fa[set][i] = *reinterpret_cast<const v4i*>(base + ra[i] * kRowBytes + ((c ^ swz(ra[i])) << 4));
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      fb[set][j] = *reinterpret_cast<const v4i*>(base + C::A_BYTES + rb[j] * kRowBytes + ((c ^ swz(rb[j])) << 4));
  };
  auto read_scales = [&](int kt) {
    const uint8_t* base = smem + (kt % STAGES) * C::STAGE;
#pragma unroll
    for (int i = 0; i < FI; ++i)
      sa[i] = (int)(*reinterpret_cast<const uint32_t*>(base + C::SA_OFF + 4 * ra[i]) >> (16 * hi));
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      sb[j] = (int)(*reinterpret_cast<const uint32_t*>(base + C::SB_OFF + 4 * rb[j]) >> (16 * hi));
  };

  v16f acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = v16f{};

  // ---- prologue: copies for steps 0 .. STAGES-2, then step 0's first half ----
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) issue(p);
  wait_vmcnt<(STAGES - 2) * C::LOADS>();
  barrier_lds();
  read_scales(0);
  read_frags(0, 0, 0);

  // One K step per iteration, in seven phases, with no branches in the body (so the
  // compiler keeps the phase order):
  //   (1) copies for step kt+STAGES-1 into the slot freed by step kt-1
  //   (2) second-half fragments of step kt
  //   (3) first-half MFMAs of step kt
  //   (4) this wave's copies of step kt+1 complete; the barrier publishes everyone's
  //   (5) first-half fragments of step kt+1
  //   (6) second-half MFMAs of step kt
  //   (7) scales of step kt+1 (the MFMAs of (6) have read the old ones at issue)
  // The MFMAs of (3) and (6) drain in the MFMA pipe while the wave waits at the
  // barrier and for its LDS reads.  On the last step, (5) and (7) read a slot that
  // holds a re-read copy; the values are unused.
  for (int kt = 0; kt < KT; ++kt) {
    issue(kt + STAGES - 1);
    read_frags(kt, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = mfma_fp4_32x32<0>(fa[0][i], fb[0][j], acc[i][j], sa[i], sb[j]);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(STAGES - 2) * C::LOADS>();
    barrier_lds();
    read_frags(kt + 1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = mfma_fp4_32x32<1>(fa[1][i], fb[1][j], acc[i][j], sa[i], sb[j]);
    __builtin_amdgcn_sched_barrier(0);
    read_scales(kt + 1);
  }
  // No copy may still be landing in LDS when the workgroup exits.
  wait_vmcnt<0>();

  // Epilogue: lane (hi, r32) of block (i, j) holds rows 8*(t/4) + 4*hi + t%4, column r32.
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int n = n0 + wn * WN + j * 32 + r32;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int m = m0 + wm * WM + i * 32 + 8 * (t >> 2) + 4 * hi + (t & 3);
        if (m < M && n < N) store_out<BF16>(D, (int64_t)m * N + n, acc[i][j][t]);
      }
    }
}

template <int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_cfg(const FP4Args& a, hipStream_t s) {
  using C = Cfg<BM, BN, WM, WN, STAGES>;
  const int64_t tiles = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  if (tiles > INT32_MAX) return hipErrorInvalidConfiguration;
  if (a.bf16_out)
    hipLaunchKernelGGL((mxfp4_gemm_kernel<BM, BN, WM, WN, STAGES, true>), dim3((unsigned)tiles), dim3(C::NT), 0,
                       s, (int)a.M, (int)a.N, (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  else
    hipLaunchKernelGGL((mxfp4_gemm_kernel<BM, BN, WM, WN, STAGES, false>), dim3((unsigned)tiles), dim3(C::NT), 0,
                       s, (int)a.M, (int)a.N, (int)a.K, a.A, a.sfA, a.B, a.sfB, a.D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp4_gemm(const FP4Args& a, hipStream_t s) {
  const int64_t t256 = ceil_div(a.M, 256) * ceil_div(a.N, 256);
  const int64_t t128 = ceil_div(a.M, 128) * ceil_div(a.N, 128);
  if (t256 >= 256) return launch_cfg<256, 256, 128, 128, 4>(a, s);
  if (t128 >= 128) return launch_cfg<128, 128, 64, 64, 4>(a, s);
  return launch_cfg<64, 64, 32, 32, 4>(a, s);
}

}  // namespace fp4g
