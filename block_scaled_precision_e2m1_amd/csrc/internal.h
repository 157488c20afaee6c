// Internal interface between the C-ABI entry points (api.cpp) and the kernel
// launchers.  Arguments reach a launcher only after validation; every
// launcher enqueues on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4g {

struct FP4Args {            // MXFP4 / NVFP4 / GEMV
  int64_t M, N, K;
  const uint8_t* A;         // [M][K/2]
  const uint8_t* sfA;       // [M][K/V]
  const uint8_t* B;         // [N][K/2]
  const uint8_t* sfB;       // [N][K/V]
  float gscale;             // NVFP4: global_a * global_b = ldexp(gscale, gscale_exp); 1 otherwise
  void* D;                  // [M][N]
  bool bf16_out;
  int64_t L = 1;            // NVFP4: problems stored back to back (grid dimension y)
  int gscale_exp = 0;       // NVFP4: gscale is the product of the two fp32 significands and
                            // gscale_exp the sum of the exponents, so no pair of finite
                            // scales overflows or flushes before it meets the accumulator
};

// Split global_a * global_b into an fp32 significand product in [0.25, 1) (one rounding)
// and a power-of-two exponent, applied in the epilogue as ldexp(acc * m, e).
void split_global_scale(float global_a, float global_b, float* m, int* e);

struct W4A8Args {
  int64_t M, N, K;
  const uint8_t* A;         // [M][K] E4M3
  const float* sa;          // [M]
  const uint8_t* B;         // [N][K/2] INT4
  const uint16_t* sB;       // [N][K/128] bf16
  void* D;
  bool bf16_out;
  int64_t L = 1;            // problems stored back to back (grid dimension y)
};

struct Fp8bArgs {            // FP8 blockwise-scaled GEMM
  int64_t M, N, K;
  const uint8_t* A;         // [M][K] E4M3
  const float* sA;          // [M][K/128]
  const uint8_t* B;         // [N][K] E4M3
  const float* sB;          // [N][K/128]
  void* D;
  bool bf16_out;
};

// Compute units of the current device (queried once per device, then cached).
int64_t device_cus();

hipError_t launch_mxfp4_gemm(const FP4Args& a, hipStream_t s);
// Batched MXFP4 GEMM: L problems of a.M x a.N x a.K stored back to back.  With S > 1
// the K stages are split S ways into the fp32 buffer P [L][S][M][N], then reduced
// into a.D in slice order; S must come from mxfp4_gemm_splits.
constexpr int64_t kMaxSplits = 16;
hipError_t launch_mxfp4_gemm_batched(const FP4Args& a, int64_t L, int64_t S, float* P, hipStream_t s);
// The K split the batched launcher uses: `requested` slices if > 0, else its own
// choice for the current device; at most `cap`, kMaxSplits and the K stage count.
int64_t mxfp4_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap);
hipError_t launch_nvfp4_gemm(const FP4Args& a, hipStream_t s);
// K-split NVFP4: nvfp4_gemm_splits gives the slice count S the launcher uses (as for
// w4a8_gemm_splits); with S > 1 the partial products go to P [L][S][M][N].  Shapes the
// decode kernel takes (nvfp4_gemv_fits) run it (no split, P unused).
int64_t nvfp4_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap);
hipError_t launch_nvfp4_gemm_split(const FP4Args& a, int64_t splits, float* P, hipStream_t s);
// NVFP4 decode GEMV for 1 <= M <= 16 tokens and K <= 16384, or 17 <= M <= 32 and
// K <= 8192 (nvfp4_gemv_fits); batch a.L.
bool nvfp4_gemv_fits(int64_t M, int64_t K);
hipError_t launch_nvfp4_gemv(const FP4Args& a, hipStream_t s);
// MXFP4 decode GEMV (L = 1) for 1 <= M <= 16 tokens, or 17 <= M <= 32 and K <= 16384.
bool fp4_gemv_fits(int64_t M, int64_t K);
hipError_t launch_fp4_gemv(const FP4Args& a, hipStream_t s);
// Pre-packed decode weights: sizes, the load-time re-pack, and the GEMV over them
// (a.B is the packed weight buffer; Sp the packed scale dwords).
void gemv_prepack_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes);
hipError_t launch_gemv_prepack(int64_t N, int64_t K, const uint8_t* B, const uint8_t* sfB, uint8_t* Bp,
                               uint32_t* Sp, hipStream_t s);
hipError_t launch_fp4_gemv_prepacked(const FP4Args& a, const uint32_t* Sp, hipStream_t s);
hipError_t launch_w4a8_gemm(const W4A8Args& a, hipStream_t s);
// Pre-packed W4A8 weights: sizes, the load-time re-pack, and the GEMM over them
// (a.B is the packed weight buffer, a.sB unused; Sp the packed fp32 scales).
void w4a8_prepack_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes);
// The fp32 group scales Sp [K/128][16*ceil(N/16)] alone (rows past N 0).
hipError_t launch_w4a8_prepack_scales(int64_t N, int64_t K, const uint16_t* sB, float* Sp, hipStream_t s);
// FP6 (E3M2) re-encoded W4A8 weights: sizes, the re-pack (weights and Sp), and the GEMM.
void w4a8_prepack_fp6_sizes(int64_t N, int64_t K, int64_t* weight_bytes, int64_t* scale_bytes);
hipError_t launch_w4a8_prepack_fp6(int64_t N, int64_t K, const uint8_t* B, const uint16_t* sB, uint8_t* Bp6,
                                   float* Sp, hipStream_t s);
bool w4a8_fp6_fits(int64_t K);             // K <= 2^23
// K split of the FP6 GEMM (128 x 128 tiles): the slice count S (`requested` if > 0, else
// the library's choice; at most `cap` and kMaxSplits), and the launcher: S > 1 writes
// the partial products to P [S][M][N] and folds them into a.D with launch_scaled_reduce.
int64_t w4a8_fp6_splits(int64_t M, int64_t N, int64_t K, int64_t requested, int64_t cap);
hipError_t launch_w4a8_gemm_prepacked_fp6_split(const W4A8Args& a, const float* Sp, int64_t splits, float* P,
                                                hipStream_t s);
hipError_t launch_w4a8_gemm_prepacked_fp6(const W4A8Args& a, const float* Sp, hipStream_t s);
hipError_t launch_w4a8_prepack(int64_t N, int64_t K, const uint8_t* B, const uint16_t* sB, uint8_t* Bp, float* Sp,
                               hipStream_t s);
hipError_t launch_w4a8_prepack_e4m3(int64_t N, int64_t K, const uint8_t* B, const uint8_t* sB8, int stride,
                                    uint8_t* Bp, float* Sp, hipStream_t s);
hipError_t launch_w4a8_gemm_prepacked(const W4A8Args& a, const float* Sp, hipStream_t s);
// The same ring kernel on plain INT4 weights and bf16 scales (K % 256 == 0, sB 4-byte aligned).
hipError_t launch_w4a8_ring(const W4A8Args& a, hipStream_t s);
// K-split W4A8 (the ring kernel; plain weights need K % 256 == 0): w4a8_gemm_splits gives
// the slice count S the launcher uses (`requested` slices if > 0, else its own choice;
// at most `cap` and kMaxSplits); with S > 1 the partial products go to the fp32 buffer
// P [L][S][M][N] and launch_scaled_reduce folds them into a.D.  Sp non-null: pre-packed
// weights (L = 1).  Shapes the decode kernel takes (w4a8_gemv_fits) run it (no split,
// P unused).
int64_t w4a8_gemm_splits(int64_t L, int64_t M, int64_t N, int64_t K, bool packed, int64_t requested, int64_t cap);
hipError_t launch_w4a8_gemm_split(const W4A8Args& a, const float* Sp, int64_t splits, float* P, hipStream_t s);
// D[b][m][n] = ldexp((sum_s P[b][s][m][n]) * (rs ? rs[b][m] : 1) * gm, ge), slices in order.
hipError_t launch_scaled_reduce(int64_t L, int64_t M, int64_t N, int S, const float* P, const float* rs, float gm,
                                int ge, void* D, bool bf16_out, hipStream_t s);
// Decode GEMV for 1 <= M <= 16 tokens and K <= 16384, or 17 <= M <= 32, K <= 8192 and
// K/128 even (w4a8_gemv_fits): weights in the 16-row slot of the FP8 instruction, tokens
// padded to one or two 16-token tiles.  Sp null: plain weights and
// bf16 scales (a.B, a.sB, batch a.L); otherwise a.B is the pre-packed weight buffer and
// Sp its fp32 scales.
bool w4a8_gemv_fits(int64_t M, int64_t K);
hipError_t launch_w4a8_gemv(const W4A8Args& a, const float* Sp, hipStream_t s);
hipError_t launch_fp8b_gemm(const Fp8bArgs& a, hipStream_t s);
// Library-held scratch (scratch.hip): kScratchBytes of device memory per GPU, for the
// allocation-free split-K entry point.  scratch_pointer returns the current device's
// address of it (looked up once per device; never the array's host-side name).
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
hipError_t scratch_pointer(float** out);
// D[M][N] = 0 (the empty-K product); never uses hipMemset so it can be captured.
hipError_t launch_zero_fill(void* D, int64_t count, bool bf16_out, hipStream_t s);
// E2M1 codes + E8M0 scales of X[rows][K] (K % 32 == 0), max-abs rule.
hipError_t launch_mx_quantize(int64_t rows, int64_t K, const void* X, bool bf16_in, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_nv_quantize(int64_t rows, int64_t K, const void* X, bool bf16_in, float g, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);

}  // namespace fp4g
