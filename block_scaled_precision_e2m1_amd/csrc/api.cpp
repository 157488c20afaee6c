// C-ABI entry points: validate on the host, pick a kernel, launch on the
// caller's stream.  Validation runs before any HIP call, so an invalid call
// returns its status without touching the device.
#include "../../include/fp4gemm.h"
#include "internal.h"

#include <stdint.h>

#include <cmath>

namespace {

using fp4g::FP4Args;
using fp4g::W4A8Args;
using fp4g::Fp8bArgs;

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // each of M, N, K below 2^31
// Output elements (L*M*N) at most 2^50: far past any device memory, and small enough
// that every byte count below (times 4 bytes, times up to 16 split slices) fits int64.
constexpr int64_t kMaxOut = (int64_t)1 << 50;
// Batches of the NVFP4 and W4A8 GEMMs are a grid dimension of at most 65535.
constexpr int64_t kMaxGridY = 65535;

struct Range { uintptr_t lo, hi; };

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared shape / pointer checks.  `out_elem` is 4 (fp32) or 2 (bf16).
// Returns FP4G_OK, or the first failing status.  `*empty` is set when the
// output has no elements (nothing to launch).
fp4g_status check_common(int64_t M, int64_t N, int64_t K, int d_type, const void* D, bool* empty) {
  if (M < 0 || N < 0 || K < 0) return FP4G_EINVAL;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (N > 0 && M > kMaxOut / N) return FP4G_EINVAL;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  *empty = (M == 0 || N == 0);
  if (*empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  return FP4G_OK;
}

fp4g_status check_fp4_operands(int64_t M, int64_t N, int64_t K, int V, const void* A, const void* sfA,
                               const void* B, const void* sfB, const void* D, int d_type) {
  if (K == 0) return FP4G_OK;                       // empty sum: inputs are not read
  if (!A || !sfA || !B || !sfB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(sfB, 4)) return FP4G_EALIGN;
  const int64_t out_bytes = M * N * (d_type == FP4G_OUT_BF16 ? 2 : 4);
  const Range d = range_of(D, out_bytes);
  const Range ins[4] = {range_of(A, M * (K / 2)), range_of(sfA, M * (K / V)),
                        range_of(B, N * (K / 2)), range_of(sfB, N * (K / V))};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  return FP4G_OK;
}

fp4g_status finish(hipError_t e) { return e == hipSuccess ? FP4G_OK : FP4G_EHIP; }

fp4g_status run_fp4(int which, int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                    float ga, float gb, const void* B, const void* sfB, void* D, int d_type, void* stream) {
  const int V = (which == 1) ? 16 : 32;
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  if (which == 2 && !fp4g::fp4_gemv_fits(M, K)) return FP4G_EUNSUPPORTED;
  st = check_fp4_operands(M, N, K, V, A, sfA, B, sfB, D, d_type);
  if (st != FP4G_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB), 1.0f, D, bf16};
  if (which == 1) fp4g::split_global_scale(ga, gb, &a.gscale, &a.gscale_exp);
  if (which == 0) return finish(fp4g::launch_mxfp4_gemm(a, s));
  if (which == 1) return finish(fp4g::launch_nvfp4_gemm(a, s));
  return finish(fp4g::launch_fp4_gemv(a, s));
}

// Sizes of the batched MXFP4 GEMM; *empty when there is no output element.
fp4g_status check_batched_sizes(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits, bool* empty) {
  if (L < 0 || L >= kMaxDim || splits < 0) return FP4G_EINVAL;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (L * M >= kMaxDim || L * N >= kMaxDim) return FP4G_EINVAL;
  if (N > 0 && L * M > kMaxOut / N) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  *empty = (L == 0 || M == 0 || N == 0);
  return FP4G_OK;
}


// The K split of a call: `requested` (0 automatic, 1 none, s > 1 at most s) limited to
// what `workspace_bytes` holds at per_split bytes a slice; the workspace is checked
// against the output and the inputs.  *S = 1 when nothing is split.
// kind 0 W4A8 plain, 1 W4A8 pre-packed, 2 NVFP4, 3 W4A8 over FP6 weights
struct SplitCtx { int64_t L, M, N, K, requested; int kind; };

int64_t choose_split(const SplitCtx& c, int64_t cap) {
  if (c.kind == 2) return fp4g::nvfp4_gemm_splits(c.L, c.M, c.N, c.K, c.requested, cap);
  if (c.kind == 3) return fp4g::w4a8_fp6_splits(c.M, c.N, c.K, c.requested, cap);
  return fp4g::w4a8_gemm_splits(c.L, c.M, c.N, c.K, c.kind == 1, c.requested, cap);
}

fp4g_status split_of(const SplitCtx& c, int64_t per_split, void* workspace, size_t workspace_bytes, const Range& d,
                     const Range* ins, int n_ins, int64_t* S) {
  *S = 1;
  if (c.requested == 1 || workspace_bytes == 0 || per_split == 0) return FP4G_OK;
  if (!aligned(workspace, 16)) return FP4G_EALIGN;
  const Range w = range_of(workspace, (int64_t)workspace_bytes);
  if (overlaps(w, d)) return FP4G_EINVAL;
  for (int i = 0; i < n_ins; ++i)
    if (overlaps(w, ins[i])) return FP4G_EINVAL;
  *S = choose_split(c, (int64_t)(workspace_bytes / (size_t)per_split));
  return FP4G_OK;
}

fp4g_status split_workspace_size(int kind, int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits,
                                 size_t* bytes) {
  bool empty = false;
  const fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (!bytes) return FP4G_EINVAL;
  *bytes = 0;
  if (empty || K == 0 || splits == 1) return FP4G_OK;
  const int64_t S = choose_split(SplitCtx{L, M, N, K, splits, kind}, fp4g::kMaxSplits);
  if (S > 1) *bytes = (size_t)(L * S * M * N * 4);
  return FP4G_OK;
}

}  // namespace

extern "C" {

fp4g_status nv_fp4_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                                float global_a, const void* B, const void* sfB, float global_b, void* D,
                                int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, 0, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (L > kMaxGridY) return FP4G_EUNSUPPORTED;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sfA || !B || !sfB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(sfB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * (K / 2)), range_of(sfA, L * M * (K / 16)),
                        range_of(B, L * N * (K / 2)), range_of(sfB, L * N * (K / 16))};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB), 1.0f, D, bf16, L};
  fp4g::split_global_scale(global_a, global_b, &a.gscale, &a.gscale_exp);
  return finish(fp4g::launch_nvfp4_gemm(a, s));
}

fp4g_status w4a8_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                              const void* B, const void* sB, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, 0, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (L > kMaxGridY) return FP4G_EUNSUPPORTED;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sa || !B || !sB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4) || !aligned(sB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * K), range_of(sa, L * M * 4), range_of(B, L * N * (K / 2)),
                        range_of(sB, L * N * (K / 128) * 2)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(B),
             static_cast<const uint16_t*>(sB), D, bf16, L};
  return finish(fp4g::launch_w4a8_gemm(a, s));
}

fp4g_status mx_fp4_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits, size_t* bytes) {
  bool empty = false;
  const fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (!bytes) return FP4G_EINVAL;
  *bytes = 0;
  if (empty || K == 0 || splits == 1) return FP4G_OK;
  const int64_t S = fp4g::mxfp4_gemm_splits(L, M, N, K, splits, fp4g::kMaxSplits);
  if (S > 1) *bytes = (size_t)(L * S * M * N * 4);
  return FP4G_OK;
}

fp4g_status mx_fp4_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                                const void* B, const void* sfB, void* D, int d_type, int64_t splits,
                                void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (!workspace && workspace_bytes > 0) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sfA || !B || !sfB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(sfB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * (K / 2)), range_of(sfA, L * M * (K / 32)),
                        range_of(B, L * N * (K / 2)), range_of(sfB, L * N * (K / 32))};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  // The split: what was asked (or chosen), limited to what the workspace holds.
  int64_t S = 1;
  if (splits != 1 && workspace_bytes > 0) {
    if (!aligned(workspace, 16)) return FP4G_EALIGN;
    const Range w = range_of(workspace, (int64_t)workspace_bytes);
    if (overlaps(w, d)) return FP4G_EINVAL;
    for (const Range& r : ins)
      if (overlaps(w, r)) return FP4G_EINVAL;
    const int64_t per_split = L * M * N * 4;
    const int64_t fits = (int64_t)(workspace_bytes / (size_t)per_split);
    S = fp4g::mxfp4_gemm_splits(L, M, N, K, splits, fits);
  }
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB), 1.0f, D, bf16};
  return finish(fp4g::launch_mxfp4_gemm_batched(a, L, S, static_cast<float*>(workspace), s));
}

fp4g_status mx_fp4_gemm_batched_noalloc(int64_t L, int64_t M, int64_t N, int64_t K, const void* A,
                                        const void* sfA, const void* B, const void* sfB, void* D,
                                        int d_type, int64_t splits, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sfA || !B || !sfB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(sfB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * (K / 2)), range_of(sfA, L * M * (K / 32)),
                        range_of(B, L * N * (K / 2)), range_of(sfB, L * N * (K / 32))};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  // The split: an explicit request must fit the library's scratch (rejected otherwise);
  // the automatic choice is limited to what fits.
  const int64_t per_split = L * M * N * 4;
  const int64_t fits = fp4g::kScratchBytes / per_split;
  int64_t S = 1;
  if (splits > 1) {
    S = fp4g::mxfp4_gemm_splits(L, M, N, K, splits, fp4g::kMaxSplits);
    if (S > 1 && S > fits) return FP4G_EUNSUPPORTED;
  } else if (splits == 0) {
    S = fp4g::mxfp4_gemm_splits(L, M, N, K, 0, fits);
  }
  float* P = nullptr;
  if (S > 1) {
    const hipError_t e = fp4g::scratch_pointer(&P);
    if (e != hipSuccess || !P) return FP4G_EHIP;
  }
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB), 1.0f, D, bf16};
  return finish(fp4g::launch_mxfp4_gemm_batched(a, L, S, P, s));
}

fp4g_status mx_fp4_gemm(int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                        const void* B, const void* sfB, void* D, int d_type, void* stream) {
  return run_fp4(0, M, N, K, A, sfA, 1.0f, 1.0f, B, sfB, D, d_type, stream);
}

fp4g_status nv_fp4_gemm(int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                        float global_a, const void* B, const void* sfB, float global_b, void* D,
                        int d_type, void* stream) {
  return run_fp4(1, M, N, K, A, sfA, global_a, global_b, B, sfB, D, d_type, stream);
}

fp4g_status fp4_gemv(int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                     const void* B, const void* sfB, void* D, int d_type, void* stream) {
  return run_fp4(2, M, N, K, A, sfA, 1.0f, 1.0f, B, sfB, D, d_type, stream);
}

fp4g_status w4a8_gemm(int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                      const void* B, const void* sB, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!A || !sa || !B || !sB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4) || !aligned(sB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sa, M * 4), range_of(B, N * (K / 2)),
                        range_of(sB, N * (K / 128) * 2)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(B),
             static_cast<const uint16_t*>(sB), D, bf16};
  return finish(fp4g::launch_w4a8_gemm(a, s));
}

fp4g_status fp8_blockwise_gemm(int64_t M, int64_t N, int64_t K, const void* A, const float* sA, const void* B,
                               const float* sB, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!A || !sA || !B || !sB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sA, 4) || !aligned(sB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sA, M * (K / 128) * 4), range_of(B, N * K),
                        range_of(sB, N * (K / 128) * 4)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  Fp8bArgs a{M, N, K, static_cast<const uint8_t*>(A), sA, static_cast<const uint8_t*>(B), sB, D, bf16};
  return finish(fp4g::launch_fp8b_gemm(a, s));
}

fp4g_status fp4_gemv_prepack_size(int64_t N, int64_t K, size_t* weight_bytes, size_t* scale_bytes) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (!weight_bytes || !scale_bytes) return FP4G_EINVAL;
  int64_t wb = 0, sb = 0;
  fp4g::gemv_prepack_sizes(N, K, &wb, &sb);
  *weight_bytes = (size_t)wb;
  *scale_bytes = (size_t)sb;
  return FP4G_OK;
}

fp4g_status fp4_gemv_prepack(int64_t N, int64_t K, const void* B, const void* sfB, void* Bp, void* Sp,
                             void* stream) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (N == 0 || K == 0) return FP4G_OK;
  if (!B || !sfB || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(B, 16) || !aligned(Bp, 16) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::gemv_prepack_sizes(N, K, &wb, &sb);
  const Range ib = range_of(B, N * (K / 2)), is = range_of(sfB, N * (K / 32));
  const Range ob = range_of(Bp, wb), os = range_of(Sp, sb);
  if (overlaps(ob, os) || overlaps(ob, ib) || overlaps(ob, is) || overlaps(os, ib) || overlaps(os, is))
    return FP4G_EINVAL;
  return finish(fp4g::launch_gemv_prepack(N, K, static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB),
                                          static_cast<uint8_t*>(Bp), static_cast<uint32_t*>(Sp),
                                          reinterpret_cast<hipStream_t>(stream)));
}

fp4g_status fp4_gemv_prepacked(int64_t M, int64_t N, int64_t K, const void* A, const void* sfA, const void* Bp,
                               const void* Sp, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  if (M > 16) return FP4G_EUNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!A || !sfA || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(Bp, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::gemv_prepack_sizes(N, K, &wb, &sb);
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * (K / 2)), range_of(sfA, M * (K / 32)), range_of(Bp, wb),
                        range_of(Sp, sb)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(Bp), nullptr, 1.0f, D, bf16};
  return finish(fp4g::launch_fp4_gemv_prepacked(a, static_cast<const uint32_t*>(Sp), s));
}

fp4g_status w4a8_prepack_size(int64_t N, int64_t K, size_t* weight_bytes, size_t* scale_bytes) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (!weight_bytes || !scale_bytes) return FP4G_EINVAL;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_sizes(N, K, &wb, &sb);
  *weight_bytes = (size_t)wb;
  *scale_bytes = (size_t)sb;
  return FP4G_OK;
}

fp4g_status w4a8_prepack(int64_t N, int64_t K, const void* B, const void* sB, void* Bp, void* Sp, void* stream) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (N == 0 || K == 0) return FP4G_OK;
  if (!B || !sB || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(B, 16) || !aligned(Bp, 16) || !aligned(sB, 2) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_sizes(N, K, &wb, &sb);
  const Range ib = range_of(B, N * (K / 2)), is = range_of(sB, N * (K / 128) * 2);
  const Range ob = range_of(Bp, wb), os = range_of(Sp, sb);
  if (overlaps(ob, os) || overlaps(ob, ib) || overlaps(ob, is) || overlaps(os, ib) || overlaps(os, is))
    return FP4G_EINVAL;
  return finish(fp4g::launch_w4a8_prepack(N, K, static_cast<const uint8_t*>(B), static_cast<const uint16_t*>(sB),
                                          static_cast<uint8_t*>(Bp), static_cast<float*>(Sp),
                                          reinterpret_cast<hipStream_t>(stream)));
}

fp4g_status w4a8_prepack_e4m3(int64_t N, int64_t K, const void* B, const void* sB8, int64_t scale_stride, void* Bp,
                              void* Sp, void* stream) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (scale_stride != 1 && scale_stride != 8) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (N == 0 || K == 0) return FP4G_OK;
  if (!B || !sB8 || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(B, 16) || !aligned(Bp, 16) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_sizes(N, K, &wb, &sb);
  const Range ib = range_of(B, N * (K / 2)), is = range_of(sB8, N * (K / 128) * scale_stride);
  const Range ob = range_of(Bp, wb), os = range_of(Sp, sb);
  if (overlaps(ob, os) || overlaps(ob, ib) || overlaps(ob, is) || overlaps(os, ib) || overlaps(os, is))
    return FP4G_EINVAL;
  return finish(fp4g::launch_w4a8_prepack_e4m3(N, K, static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sB8),
                                               (int)scale_stride, static_cast<uint8_t*>(Bp), static_cast<float*>(Sp),
                                               reinterpret_cast<hipStream_t>(stream)));
}

fp4g_status w4a8_gemm_prepacked(int64_t M, int64_t N, int64_t K, const void* A, const float* sa, const void* Bp,
                                const void* Sp, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!A || !sa || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(Bp, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_sizes(N, K, &wb, &sb);
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sa, M * 4), range_of(Bp, wb), range_of(Sp, sb)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(Bp), nullptr, D, bf16};
  return finish(fp4g::launch_w4a8_gemm_prepacked(a, static_cast<const float*>(Sp), s));
}

fp4g_status w4a8_prepack_fp6_size(int64_t N, int64_t K, size_t* weight_bytes, size_t* scale_bytes) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (!weight_bytes || !scale_bytes) return FP4G_EINVAL;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_fp6_sizes(N, K, &wb, &sb);
  *weight_bytes = (size_t)wb;
  *scale_bytes = (size_t)sb;
  return FP4G_OK;
}

fp4g_status w4a8_prepack_fp6(int64_t N, int64_t K, const void* B, const void* sB, void* Bp6, void* Sp,
                             void* stream) {
  if (N < 0 || K < 0 || N >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K % 128 != 0) return FP4G_EUNSUPPORTED;
  if (N == 0 || K == 0) return FP4G_OK;
  if (!B || !sB || !Bp6 || !Sp) return FP4G_EINVAL;
  if (!aligned(B, 16) || !aligned(Bp6, 16) || !aligned(sB, 2) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_fp6_sizes(N, K, &wb, &sb);
  const Range ib = range_of(B, N * (K / 2)), is = range_of(sB, N * (K / 128) * 2);
  const Range ob = range_of(Bp6, wb), os = range_of(Sp, sb);
  if (overlaps(ob, os) || overlaps(ob, ib) || overlaps(ob, is) || overlaps(os, ib) || overlaps(os, is))
    return FP4G_EINVAL;
  return finish(fp4g::launch_w4a8_prepack_fp6(N, K, static_cast<const uint8_t*>(B), static_cast<const uint16_t*>(sB),
                                              static_cast<uint8_t*>(Bp6), static_cast<float*>(Sp),
                                              reinterpret_cast<hipStream_t>(stream)));
}

fp4g_status w4a8_gemm_prepacked_fp6(int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                                    const void* Bp6, const void* Sp, void* D, int d_type, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!fp4g::w4a8_fp6_fits(K)) return FP4G_EUNSUPPORTED;
  if (!A || !sa || !Bp6 || !Sp) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(Bp6, 16) || !aligned(Sp, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_fp6_sizes(N, K, &wb, &sb);
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sa, M * 4), range_of(Bp6, wb), range_of(Sp, sb)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(Bp6), nullptr, D, bf16};
  return finish(fp4g::launch_w4a8_gemm_prepacked_fp6(a, static_cast<const float*>(Sp), s));
}

fp4g_status mx_fp4_quantize(int64_t rows, int64_t K, const void* X, int x_type, void* codes, void* scales,
                            void* stream) {
  if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K > 0 && rows > kMaxOut / K) return FP4G_EINVAL;
  if (x_type != FP4G_IN_F32 && x_type != FP4G_IN_BF16) return FP4G_EINVAL;
  if (K % 32 != 0) return FP4G_EUNSUPPORTED;
  if (rows == 0 || K == 0) return FP4G_OK;
  if (!X || !codes || !scales) return FP4G_EINVAL;
  if (!aligned(X, 16) || !aligned(codes, 16)) return FP4G_EALIGN;
  const Range x = range_of(X, rows * K * (x_type == FP4G_IN_BF16 ? 2 : 4));
  const Range c = range_of(codes, rows * (K / 2)), sc = range_of(scales, rows * (K / 32));
  if (overlaps(x, c) || overlaps(x, sc) || overlaps(c, sc)) return FP4G_EINVAL;
  return finish(fp4g::launch_mx_quantize(rows, K, X, x_type == FP4G_IN_BF16, static_cast<uint8_t*>(codes),
                                         static_cast<uint8_t*>(scales), reinterpret_cast<hipStream_t>(stream)));
}

fp4g_status nv_fp4_quantize(int64_t rows, int64_t K, const void* X, int x_type, float global_scale, void* codes,
                            void* scales, void* stream) {
  if (rows < 0 || K < 0 || rows >= kMaxDim || K >= kMaxDim) return FP4G_EINVAL;
  if (K > 0 && rows > kMaxOut / K) return FP4G_EINVAL;
  if (x_type != FP4G_IN_F32 && x_type != FP4G_IN_BF16) return FP4G_EINVAL;
  if (!(global_scale > 0.0f) || !std::isfinite(global_scale)) return FP4G_EINVAL;
  if (K % 16 != 0) return FP4G_EUNSUPPORTED;
  if (rows == 0 || K == 0) return FP4G_OK;
  if (!X || !codes || !scales) return FP4G_EINVAL;
  if (!aligned(X, 16) || !aligned(codes, 8)) return FP4G_EALIGN;
  const Range x = range_of(X, rows * K * (x_type == FP4G_IN_BF16 ? 2 : 4));
  const Range c = range_of(codes, rows * (K / 2)), sc = range_of(scales, rows * (K / 16));
  if (overlaps(x, c) || overlaps(x, sc) || overlaps(c, sc)) return FP4G_EINVAL;
  return finish(fp4g::launch_nv_quantize(rows, K, X, x_type == FP4G_IN_BF16, global_scale,
                                         static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                         reinterpret_cast<hipStream_t>(stream)));
}

const char* fp4g_status_string(int status) {
  switch (status) {
    case FP4G_OK: return "ok";
    case FP4G_EINVAL: return "invalid argument (null pointer, negative size, bad output type or D overlapping an input)";
    case FP4G_EUNSUPPORTED: return "unsupported shape (K must be a multiple of 128, of 32 for the MX quantizer, of 16 for the NV quantizer; GEMV needs M <= 16, or M <= 32 with K <= 16384; the pre-packed GEMV M <= 16)";
    case FP4G_EALIGN: return "misaligned pointer (operands and D need 16-byte, scales 4-byte alignment)";
    case FP4G_EHIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
  }
}

fp4g_status w4a8_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits, size_t* bytes) {
  // the larger of the two weight forms' needs (pre-packed weights also split K % 256 != 0)
  return split_workspace_size(1, L, M, N, K, splits, bytes);
}

fp4g_status nv_fp4_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits, size_t* bytes) {
  return split_workspace_size(2, L, M, N, K, splits, bytes);
}

fp4g_status w4a8_gemm_split(int64_t L, int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                            const void* B, const void* sB, void* D, int d_type, int64_t splits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (L > kMaxGridY) return FP4G_EUNSUPPORTED;
  if (!workspace && workspace_bytes > 0) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sa || !B || !sB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4) || !aligned(sB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * K), range_of(sa, L * M * 4), range_of(B, L * N * (K / 2)),
                        range_of(sB, L * N * (K / 128) * 2)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  int64_t S = 1;
  st = split_of(SplitCtx{L, M, N, K, splits, 0}, L * M * N * 4, workspace, workspace_bytes, d, ins, 4, &S);
  if (st != FP4G_OK) return st;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(B),
             static_cast<const uint16_t*>(sB), D, bf16, L};
  if (S > 1) return finish(fp4g::launch_w4a8_gemm_split(a, nullptr, S, static_cast<float*>(workspace), s));
  return finish(fp4g::launch_w4a8_gemm(a, s));
}

fp4g_status w4a8_gemm_prepacked_split(int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                                      const void* Bp, const void* Sp, void* D, int d_type, int64_t splits,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK) return st;
  if (splits < 0) return FP4G_EINVAL;
  if (!workspace && workspace_bytes > 0) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!A || !sa || !Bp || !Sp) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(Bp, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4) || !aligned(Sp, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_sizes(N, K, &wb, &sb);
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sa, M * 4), range_of(Bp, wb), range_of(Sp, sb)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  int64_t S = 1;
  st = split_of(SplitCtx{1, M, N, K, splits, 1}, M * N * 4, workspace, workspace_bytes, d, ins, 4, &S);
  if (st != FP4G_OK) return st;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(Bp), nullptr, D, bf16};
  return finish(fp4g::launch_w4a8_gemm_split(a, static_cast<const float*>(Sp), S,
                                             S > 1 ? static_cast<float*>(workspace) : nullptr, s));
}

fp4g_status w4a8_fp6_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits, size_t* bytes) {
  return split_workspace_size(3, 1, M, N, K, splits, bytes);
}

fp4g_status w4a8_gemm_prepacked_fp6_split(int64_t M, int64_t N, int64_t K, const void* A, const float* sa,
                                          const void* Bp6, const void* Sp, void* D, int d_type, int64_t splits,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  fp4g_status st = check_common(M, N, K, d_type, D, &empty);
  if (st != FP4G_OK) return st;
  if (splits < 0) return FP4G_EINVAL;
  if (!workspace && workspace_bytes > 0) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf16 = d_type == FP4G_OUT_BF16;
  if (K == 0) return finish(fp4g::launch_zero_fill(D, M * N, bf16, s));
  if (!fp4g::w4a8_fp6_fits(K)) return FP4G_EUNSUPPORTED;
  if (!A || !sa || !Bp6 || !Sp) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(Bp6, 16) || !aligned(Sp, 16)) return FP4G_EALIGN;
  if (!aligned(sa, 4)) return FP4G_EALIGN;
  int64_t wb = 0, sb = 0;
  fp4g::w4a8_prepack_fp6_sizes(N, K, &wb, &sb);
  const Range d = range_of(D, M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, M * K), range_of(sa, M * 4), range_of(Bp6, wb), range_of(Sp, sb)};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  int64_t S = 1;
  st = split_of(SplitCtx{1, M, N, K, splits, 3}, M * N * 4, workspace, workspace_bytes, d, ins, 4, &S);
  if (st != FP4G_OK) return st;
  W4A8Args a{M, N, K, static_cast<const uint8_t*>(A), sa, static_cast<const uint8_t*>(Bp6), nullptr, D, bf16};
  return finish(fp4g::launch_w4a8_gemm_prepacked_fp6_split(a, static_cast<const float*>(Sp), S,
                                                           S > 1 ? static_cast<float*>(workspace) : nullptr, s));
}

fp4g_status nv_fp4_gemm_split(int64_t L, int64_t M, int64_t N, int64_t K, const void* A, const void* sfA,
                              float global_a, const void* B, const void* sfB, float global_b, void* D, int d_type,
                              int64_t splits, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  fp4g_status st = check_batched_sizes(L, M, N, K, splits, &empty);
  if (st != FP4G_OK) return st;
  if (d_type != FP4G_OUT_F32 && d_type != FP4G_OUT_BF16) return FP4G_EINVAL;
  if (L > kMaxGridY) return FP4G_EUNSUPPORTED;
  if (!workspace && workspace_bytes > 0) return FP4G_EINVAL;
  if (empty) return FP4G_OK;
  if (!D) return FP4G_EINVAL;
  if (!aligned(D, 16)) return FP4G_EALIGN;
  const bool bf16 = d_type == FP4G_OUT_BF16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) return finish(fp4g::launch_zero_fill(D, L * M * N, bf16, s));
  if (!A || !sfA || !B || !sfB) return FP4G_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16)) return FP4G_EALIGN;
  if (!aligned(sfA, 4) || !aligned(sfB, 4)) return FP4G_EALIGN;
  const Range d = range_of(D, L * M * N * (bf16 ? 2 : 4));
  const Range ins[4] = {range_of(A, L * M * (K / 2)), range_of(sfA, L * M * (K / 16)),
                        range_of(B, L * N * (K / 2)), range_of(sfB, L * N * (K / 16))};
  for (const Range& r : ins)
    if (overlaps(d, r)) return FP4G_EINVAL;
  int64_t S = 1;
  st = split_of(SplitCtx{L, M, N, K, splits, 2}, L * M * N * 4, workspace, workspace_bytes, d, ins, 4, &S);
  if (st != FP4G_OK) return st;
  FP4Args a{M, N, K, static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(sfA),
            static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(sfB), 1.0f, D, bf16, L};
  fp4g::split_global_scale(global_a, global_b, &a.gscale, &a.gscale_exp);
  return finish(fp4g::launch_nvfp4_gemm_split(a, S, S > 1 ? static_cast<float*>(workspace) : nullptr, s));
}

}  // extern "C"
