/*
 * fp4gemm.h -- C ABI of the block-scaled FP4 GEMM library for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (all entry points): an output tile D[M][N] of
 *   D[m][n] = sum_k  (a[m][k] * sa[m][k / V]) * (b[n][k] * sb[n][k / V])
 * where a, b are 4-bit E2M1 codes and sa, sb block scales, one per V
 * consecutive K elements.  The block-scaled MMA and its scale granularity are
 * the subject of the NVIDIA/cutlass issue "Add FP4 TMA kernel example for
 * Blackwell in CuTe Python DSL" (sections "What Works", "MMA Instruction K
 * Constraint", "Scale Factor Granularity" and "Code Reference"); the MXFP4
 * variant with E8M0 scales is section 1 of the cuda-oxide page "TMA
 * Pipelines, Tensor Cores, and ctm-rs Interop"; the W4A8 variant is the
 * Hopper CUTLASS/CuTe DSL blog post, sections "The W4A8 kernel: the same four
 * definitions, with the operands swapped" and "What changes in the W4A8
 * builder".
 *
 * Layouts (normative; every pointer is device memory owned by the caller):
 *   FP4 / INT4 operand  X[rows][K/2] bytes, row-major (K contiguous, "K-major"
 *                       for both operands); the low nibble of byte j holds
 *                       element 2j, the high nibble element 2j+1.
 *   E2M1 nibble         sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *                       values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   MX scales           sf[rows][K/32] bytes, row-major; E8M0: value 2^(e-127),
 *                       0xFF is NaN.
 *   NV scales           sf[rows][K/16] bytes, row-major; E4M3 (OCP "FN": bias 7,
 *                       max 448, 0x7F/0xFF NaN, no infinities).
 *   W4A8 activations    A[M][K] bytes, E4M3 codes; row scales sa[M] fp32.
 *   W4A8 weights        B[N][K/2] bytes, two's-complement INT4 nibbles
 *                       (-8..7); group scales sB[N][K/128] bf16.
 *   Output              D[M][N] row-major (leading dimension N), fp32 or bf16
 *                       (round to nearest even).  D is only written, never read.
 *
 * Calls are asynchronous: each entry point validates its arguments on the
 * host, then enqueues its kernel on `stream` (a hipStream_t; NULL is the
 * default stream) and returns.  Faults inside a kernel surface at the
 * caller's next synchronisation.  The library allocates no memory and keeps no
 * per-call state.  The only state it keeps is per device and set on first use:
 * the compute-unit count (queried once, to size grids), and, for
 * mx_fp4_gemm_batched_noalloc, the address of its scratch array.  Entry points
 * may be called from several threads at once, except that calls of
 * mx_fp4_gemm_batched_noalloc that overlap on one GPU share its scratch.
 * Validation failures return a status code and launch nothing.
 *
 * Sizes (all entry points): M, N, K >= 0 and below 2^31, and M*N (L*M*N for
 * the batched GEMM) at most 2^50 (FP4G_EINVAL otherwise); K a multiple of 128
 * (FP4G_EUNSUPPORTED otherwise).  M == 0 or N == 0 is an empty output: nothing
 * is read, written or launched, and the call returns FP4G_OK.  K == 0 is an
 * empty sum: D is set to zero and the inputs are not read (they may be NULL).
 */
#ifndef FP4GEMM_H
#define FP4GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP4G_OK = 0,
    FP4G_EINVAL = 1,       /* null pointer, negative or too large size, bad enum, D overlaps an input */
    FP4G_EUNSUPPORTED = 2, /* K not a multiple of 128 (of 32 for the quantizer), or GEMV with M > 32
                              (M > 16 with K > 16384; the pre-packed GEMV M > 16) */
    FP4G_EALIGN = 3,       /* operand / output not 16-byte aligned, scales not 4-byte aligned */
    FP4G_EHIP = 4          /* the HIP runtime rejected the launch */
} fp4g_status;

/* Output type of D.  Entry points take it as `int d_type` (and the quantizers' input
 * type as `int x_type`), the enums' underlying type: callers from C, ctypes and other
 * foreign-function layers may pass any int, every value is validated
 * (FP4G_EINVAL unless it names an enumerator), and in the C++ implementation an enum
 * parameter holding a value outside its enumerators would be undefined. */
typedef enum {
    FP4G_OUT_F32 = 0,
    FP4G_OUT_BF16 = 1
} fp4g_out;

typedef enum {
    FP4G_IN_F32 = 0,
    FP4G_IN_BF16 = 1
} fp4g_in;

/* MXFP4 GEMM: V = 32, E8M0 scales.
 *   A [M][K/2], sfA [M][K/32], B [N][K/2], sfB [N][K/32], D [M][N] of d_type.
 * With 1 <= M <= 32 in fp4_gemv's range and K >= 4096 (also mx_fp4_gemm_batched with
 * L = 1 and its automatic split) it runs the decode GEMV kernel; the result bar is the
 * same. */
fp4g_status mx_fp4_gemm(int64_t M, int64_t N, int64_t K,
                        const void *A, const void *sfA,
                        const void *B, const void *sfB,
                        void *D, int d_type, void *stream);

/* Batched MXFP4 GEMM with an optional split of K.  The problem shape is
 * (M, N, K, L), L the batch count, all four runtime values (the Hopper
 * CUTLASS/CuTe DSL blog post, section "How a kernel is assembled"): L
 * independent MXFP4 products of one shape, stored back to back:
 *   A [L][M][K/2], sfA [L][M][K/32], B [L][N][K/2], sfB [L][N][K/32],
 *   D [L][M][N] of d_type.
 * When the output tiles are too few to fill the GPU (skinny or small problems;
 * the post's introduction names a stream-K scheduler as the load-balancing
 * variant of the persistent one), the K loop is cut into s slices whose fp32
 * partial sums go to `workspace` and are then added in slice order.
 *   splits     0: the library chooses s for the current device; 1: no split;
 *              s > 1: s slices.  s is clamped to 16, to the number of K stages
 *              (K/256 when K % 256 == 0, else K/128) and to what the workspace
 *              holds; below 2 nothing is split.
 *   workspace  caller-owned device memory of workspace_bytes (16-byte aligned,
 *              not overlapping any input or D), or NULL with 0 bytes.  A split
 *              into s slices uses L*s*M*N*4 bytes.  Its contents on entry are
 *              ignored and on return undefined; calls in flight at the same time
 *              must not share a workspace.
 * For a given s the result is reproducible bit for bit; different s round
 * differently, each within fp32 accumulation error.  L == 0 behaves like
 * M == 0; L < 0 or L*M, L*N >= 2^31 is FP4G_EINVAL.  With L == 1 and no split
 * this is mx_fp4_gemm. */
fp4g_status mx_fp4_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K,
                                const void *A, const void *sfA,
                                const void *B, const void *sfB,
                                void *D, int d_type, int64_t splits,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Workspace that mx_fp4_gemm_batched with these sizes and `splits` uses on the
 * current device when given as much as it wants: L*s*M*N*4 bytes for the split s
 * it would pick, 0 when it would not split.  Writes *bytes; sizes are checked as
 * in mx_fp4_gemm_batched (FP4G_EINVAL, FP4G_EUNSUPPORTED; bytes may not be NULL). */
fp4g_status mx_fp4_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K,
                                       int64_t splits, size_t *bytes);

/* mx_fp4_gemm_batched for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, layouts, kernels and results, with no workspace argument.  A split of K
 * keeps its fp32 partial sums in a scratch array that the library holds in every GPU's
 * memory it runs on (32 MiB per GPU, until the process ends; its address is looked up
 * once per device on the first call with that device current).  The call allocates
 * nothing.
 *   splits  0: the library chooses s, limited to what the scratch holds
 *           (L*s*M*N*4 <= 32 MiB); 1: no split; s > 1: s slices (clamped to 16 and to
 *           the number of K stages as in mx_fp4_gemm_batched), rejected with
 *           FP4G_EUNSUPPORTED when L*s*M*N*4 exceeds 32 MiB.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in time on
 * one GPU (other streams, other host threads) race on it and must be serialised by the
 * caller.  The partial sums are written in full before they are read, so nothing needs
 * clearing between calls.  Validation and other statuses as for mx_fp4_gemm_batched;
 * FP4G_EHIP also when the scratch address cannot be obtained. */
fp4g_status mx_fp4_gemm_batched_noalloc(int64_t L, int64_t M, int64_t N, int64_t K,
                                        const void *A, const void *sfA,
                                        const void *B, const void *sfB,
                                        void *D, int d_type, int64_t splits, void *stream);

/* NVFP4 GEMM: V = 16, E4M3 scales, then D *= global_a * global_b.
 *   A [M][K/2], sfA [M][K/16], B [N][K/2], sfB [N][K/16], D [M][N].
 * With 1 <= M <= 16 and K <= 16384, or 17 <= M <= 32 and K <= 8192 (also in
 * nv_fp4_gemm_batched), a decode kernel streams B once with the tokens in one or two
 * 16-wide tiles; the result bar is the same. */
fp4g_status nv_fp4_gemm(int64_t M, int64_t N, int64_t K,
                        const void *A, const void *sfA, float global_a,
                        const void *B, const void *sfB, float global_b,
                        void *D, int d_type, void *stream);

/* W4A8 mixed-input GEMM (FP8 E4M3 activations x INT4 weights):
 *   D[m][n] = sa[m] * sum_g bf16(sB[n][g]) * sum_{k in group g} e4m3(A[m][k]) * int4(B[n][k])
 *   with groups of 128 consecutive K elements.
 *   A [M][K] bytes, sa [M] fp32, B [N][K/2] bytes, sB [N][K/128] bf16 (raw
 *   16-bit patterns), D [M][N].
 * Accuracy (also for w4a8_gemm_prepacked and w4a8_gemm_batched).  The products run on
 * the scaled FP8 matrix instruction, which truncates: in every aligned run of 8
 * consecutive K elements it drops from each product the part below 2^(E - 13), E the
 * largest exponent sum e(a) + e(w) of the run's products (e = the E4M3 exponent field,
 * -6 for subnormals; measured on gfx950).  Weights enter it as the two exact parts
 * v = q mod 8 and -8 [q < 0] when K % 256 == 0 and for pre-packed weights, else as the
 * one E4M3 value q; in the decode kernel (1 <= M <= 16 with K <= 16384, or
 * 17 <= M <= 32 with K <= 8192 and K/128 even) as the same two parts with v written as
 * the subnormal code v * 2^-9 and both parts scaled back by 2^9, so that every nonzero v
 * counts with exponent field 3 in E.  With S = sum of
 * |products| and H = the sum over runs of
 * |product| mod 2^(E - 13) (every scale folded into both):
 *   |D - D_exact| <= 1e-5 * S + H       (plus one bf16 ulp of D_exact for bf16 output).
 * H is zero when the activation exponents inside every run of 8 span at most 6
 * binades; for N(0,1)-like activations scaled into the E4M3 range it stays near
 * 1e-6 * S.  Activations whose runs mix far more binades can reach H up to about
 * 8e-4 * S in the worst case (one product per run 2^14 times the others). */
fp4g_status w4a8_gemm(int64_t M, int64_t N, int64_t K,
                      const void *A, const float *sa,
                      const void *B, const void *sB,
                      void *D, int d_type, void *stream);

/* Pre-packed W4A8 weights (the load-time re-encoding and re-ordering of the
 * weights and re-packing of the scales that the Hopper CUTLASS/CuTe DSL blog post
 * describes for its fast INT4 -> FP8 conversion, section "The W4A8 kernel: the
 * same four definitions, with the operands swapped").  With G16 = ceil(N/16)
 * groups of 16 weight rows, KG = K/128 scale groups, lane = 16*slot + r:
 *   Bp bytes [G16][KG][64 lanes][16]: the 32 INT4 nibbles of row 16*g16 + r,
 *      K = 128*kg + 32*slot + 0..31, re-ordered so that byte 4*w + j holds element
 *      8*w + j in its low nibble and element 8*w + j + 4 in its high nibble
 *      (same two's-complement values);
 *   Sp fp32 [KG][16*G16]: Sp[kg][n] = sB[n][kg] widened from bf16 (exact).
 * Rows past N are zero with scale 0.
 *
 * w4a8_prepack_size: bytes of Bp (G16*KG*1024) and Sp (KG*16*G16*4); sizes as
 *   for w4a8_gemm; neither pointer may be NULL.
 * w4a8_prepack: writes Bp and Sp from B [N][K/2] and sB [N][K/128] (bf16 bits)
 *   on `stream`.  B and Bp 16-byte aligned, sB 2-byte and Sp 4-byte aligned;
 *   outputs must not overlap each other or the inputs.  N == 0 or K == 0 is a
 *   no-op.
 * w4a8_gemm_prepacked: w4a8_gemm (same A, sa and D layouts and result) with the
 *   weights given as Bp and Sp.  A 16-byte aligned, sa, Bp and Sp as above; D
 *   must not overlap any input. */
fp4g_status w4a8_prepack_size(int64_t N, int64_t K, size_t *weight_bytes, size_t *scale_bytes);
fp4g_status w4a8_prepack(int64_t N, int64_t K, const void *B, const void *sB,
                         void *Bp, void *Sp, void *stream);
fp4g_status w4a8_gemm_prepacked(int64_t M, int64_t N, int64_t K,
                                const void *A, const float *sa,
                                const void *Bp, const void *Sp,
                                void *D, int d_type, void *stream);

/* The same pre-packed weights from E4M3 group scales instead of bf16 ones: the FP8
 * scale type of the Hopper post's W4A8 kernel (section "The W4A8 kernel: the same four
 * definitions, with the operands swapped", where each FP8 scale is stored as
 * Array<float_e4m3_t, 8>).  Scale (n, g) is the E4M3 byte sB8[(n * (K/128) + g) *
 * scale_stride]: scale_stride 1 for a plain [N][K/128] array, 8 for that Array<8>
 * packing (the first of the 8 bytes is read).  Bp is as from w4a8_prepack and Sp
 * holds the scales widened to fp32 (exact; a NaN code stays NaN), so
 * w4a8_gemm_prepacked computes
 *   D[m][n] = sa[m] * sum_g e4m3(scale(n, g)) * sum_{k in g} e4m3(A[m][k]) * int4(B[n][k]).
 * scale_stride other than 1 or 8 is FP4G_EINVAL; alignment and overlap rules as for
 * w4a8_prepack (sB8 needs no alignment). */
fp4g_status w4a8_prepack_e4m3(int64_t N, int64_t K, const void *B, const void *sB8, int64_t scale_stride,
                              void *Bp, void *Sp, void *stream);

/* W4A8 weights re-encoded as FP6 at load time (the load-time re-encoding and
 * re-ordering of the Hopper CUTLASS/CuTe DSL blog post, section "The W4A8 kernel: the
 * same four definitions, with the operands swapped", taken one step further on this
 * chip): every INT4 value -8..7 is exact in the FP6 format E3M2 (sign bit 5, exponent
 * field bits 4..2 with bias 3, mantissa bits 1..0), and gfx950's scaled matrix
 * instruction multiplies E3M2 by E4M3 at the FP8 rate.  The GEMM then runs one
 * instruction per product where the INT4 kernels run two, and converts nothing.  The
 * weights take 6 bits instead of 4, so for decode (M <= 32, a weight stream) the INT4
 * forms stay faster.  With G32 = ceil(N/32), KG = K/128, lane l = 16*slot + r:
 *   Bp6 bytes [G32][KG][3072]: per block, bytes 16l..16l+15 of 0..1023 hold dwords 0-3
 *      of lane l for rows 32*g32 + r, bytes 1024 + 16l.. the same for rows 32*g32 + 16 + r,
 *      bytes 2048 + 16l.. dwords 4-5 of the first half then of the second; a lane's six
 *      dwords hold its 32 E3M2 codes, code e at bits 6e..6e+5, for
 *      K = 128*kg + 64*(slot & 1) + 16*(slot >> 1) + e + (e < 16 ? 0 : 16)
 *      (the K order in which the instruction pairs an FP6 operand with FP8 activations
 *      whose lane of slot s holds K 32s..32s+31, measured on gfx950);
 *   Sp as from w4a8_prepack (fp32 [KG][16*ceil(N/16)]).
 * Rows past N are zero codes with scale 0.
 *
 * w4a8_prepack_fp6_size: bytes of Bp6 (G32*KG*3072) and Sp; sizes as for w4a8_gemm.
 * w4a8_prepack_fp6: writes Bp6 and Sp from B and sB; alignment, overlap and empty-size
 *   rules as for w4a8_prepack.
 * w4a8_gemm_prepacked_fp6: w4a8_gemm (same A, sa and D layouts) over Bp6 and Sp.  The
 *   instruction's results equal those of the FP8 instruction on the one E4M3 value q bit
 *   for bit (measured on gfx950), so the accuracy is w4a8_gemm's for the one-value form:
 *   |D - D_exact| <= 1e-5 * S + H.  A, Bp6 and Sp 16-byte aligned, sa 4-byte; D must
 *   not overlap any input; K > 2^23 is FP4G_EUNSUPPORTED.
 * w4a8_gemm_prepacked_fp6_split: the same product with a split of K for problems whose
 *   tiles cannot fill the GPU (the fp32 partial products of the slices go to `workspace`
 *   and are then added in slice order and scaled by sa).  `splits` and `workspace` as for
 *   w4a8_gemm_prepacked_split (a slice keeps at least 2 K groups); the result is
 *   reproducible bit for bit for a given split and within the same bound.
 * w4a8_fp6_workspace_size: the workspace bytes the split call takes for these sizes and
 *   `splits` (0 when it would not split). */
fp4g_status w4a8_prepack_fp6_size(int64_t N, int64_t K, size_t *weight_bytes, size_t *scale_bytes);
fp4g_status w4a8_prepack_fp6(int64_t N, int64_t K, const void *B, const void *sB,
                             void *Bp6, void *Sp, void *stream);
fp4g_status w4a8_gemm_prepacked_fp6(int64_t M, int64_t N, int64_t K,
                                    const void *A, const float *sa,
                                    const void *Bp6, const void *Sp,
                                    void *D, int d_type, void *stream);
fp4g_status w4a8_fp6_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits, size_t *bytes);
fp4g_status w4a8_gemm_prepacked_fp6_split(int64_t M, int64_t N, int64_t K,
                                          const void *A, const float *sa,
                                          const void *Bp6, const void *Sp,
                                          void *D, int d_type, int64_t splits,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* FP8 blockwise-scaled GEMM, the FP8 starting point of the issue page ("What
 * Works"; "Scale Factor Granularity": FP8 scales cover 128 elements of K):
 *   D[m][n] = sum_g sA[m][g] * sB[n][g] * sum_{k in group g} e4m3(A[m][k]) * e4m3(B[n][k])
 *   with groups of 128 consecutive K elements and one fp32 scale per row per group.
 *   A [M][K] bytes and B [N][K] bytes of E4M3 codes (K-major), sA [M][K/128] and
 *   sB [N][K/128] fp32, D [M][N].  Scales need 4-byte alignment.
 * Accuracy: as for w4a8_gemm, |D - D_exact| <= 1e-5 * S + H with H the FP8
 * instruction's truncation over aligned runs of 8 products (|a b| mod 2^(E - 13), E the
 * run's largest exponent sum, scales folded in).  H is zero when every product of a run
 * is a multiple of its unit, for example when both operands' exponents inside every run
 * span at most 3 binades; for N(0,1) operands quantized per 128-block it stays below
 * 1e-5 * S. */
fp4g_status fp8_blockwise_gemm(int64_t M, int64_t N, int64_t K,
                               const void *A, const float *sA,
                               const void *B, const float *sB,
                               void *D, int d_type, void *stream);

/* MXFP4 GEMV for decode (few tokens): the MXFP4 GEMM with 1 <= M <= 16 (any K), or
 * 17 <= M <= 32 with K <= 16384 (a second 16-token tile over the same weight fragments),
 * and the same layouts, tuned for streaming the weight operand B once from HBM.  The
 * cute-rs page lists the MXFP4 GEMV among its next steps ("Where to Go Next"); the
 * Hopper CUTLASS/CuTe DSL blog post sizes the token tile from 16 for this decode regime
 * and swaps the operands so the weights fill the instruction's wide side (sections "What
 * changes in the W4A8 builder" and "The W4A8 kernel: the same four definitions, with
 * the operands swapped").  Other M (or M > 16 with K > 16384) return
 * FP4G_EUNSUPPORTED. */
fp4g_status fp4_gemv(int64_t M, int64_t N, int64_t K,
                     const void *A, const void *sfA,
                     const void *B, const void *sfB,
                     void *D, int d_type, void *stream);

/* Batched NVFP4 and W4A8 GEMMs: L independent problems of one shape stored back
 * to back, the same (M, N, K, L) problem shape as mx_fp4_gemm_batched (the Hopper
 * CUTLASS/CuTe DSL blog post, section "How a kernel is assembled"):
 *   NVFP4: A [L][M][K/2], sfA [L][M][K/16], B [L][N][K/2], sfB [L][N][K/16],
 *          D [L][M][N]; global_a and global_b apply to every problem.
 *   W4A8:  A [L][M][K], sa [L][M], B [L][N][K/2], sB [L][N][K/128], D [L][M][N].
 * Sizes as for mx_fp4_gemm_batched, and L <= 65535 (FP4G_EUNSUPPORTED above). */
fp4g_status nv_fp4_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K,
                                const void *A, const void *sfA, float global_a,
                                const void *B, const void *sfB, float global_b,
                                void *D, int d_type, void *stream);
fp4g_status w4a8_gemm_batched(int64_t L, int64_t M, int64_t N, int64_t K,
                              const void *A, const float *sa,
                              const void *B, const void *sB,
                              void *D, int d_type, void *stream);

/* K split for the NVFP4 and W4A8 GEMMs.  A problem with too few output tiles to fill the
 * GPU (a skinny M, a small batch) can split its K groups into S slices of consecutive
 * groups: the plain, fixed form of dividing K among workgroups, which the stream-K tile
 * scheduler of one variant of the running example in the Hopper CUTLASS/CuTe DSL blog
 * post does adaptively (its introduction); each slice writes an fp32 partial product
 * into the caller's workspace, and a second kernel sums the slices in slice order and
 * applies the per-token scales (W4A8) or global scales (NVFP4) as the unsplit epilogue
 * does.  Results meet the same accuracy bar as the unsplit calls.
 *
 * nv_fp4_gemm_split: nv_fp4_gemm_batched (same layouts, sizes and result) with a split.
 * w4a8_gemm_split: w4a8_gemm_batched (same layouts, sizes and result) with a split;
 *   plain weights split only when K % 256 == 0.
 * w4a8_gemm_prepacked_split: w4a8_gemm_prepacked (same layouts and result) with a split.
 * `splits`: 0 lets the library choose (no split when the tiles already fill the GPU), 1
 *   never splits, s > 1 asks for at most s slices; a slice keeps at least 2 K groups
 *   (W4A8: an even number), and S never exceeds 16 or what `workspace` holds.  Where
 *   the decode kernels run (1 <= M <= 16; 17 <= M <= 32 with K <= 8192, for W4A8 also
 *   K/128 even) nothing is split.
 * workspace: device memory of workspace_bytes (16-byte aligned, overlapping neither D nor
 *   any input), or NULL with workspace_bytes == 0 (no split).  S slices use L*S*M*N*4
 *   bytes, written in full before they are read: nothing needs clearing.
 * nv_fp4_gemm_workspace_size / w4a8_gemm_workspace_size: the workspace bytes the split
 *   call takes for these sizes and `splits` (0 when it would not split); the W4A8 size
 *   covers both weight forms (pass L = 1 for the pre-packed call).
 * Statuses as for the unsplit calls; splits < 0 is FP4G_EINVAL. */
fp4g_status nv_fp4_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits,
                                       size_t *bytes);
fp4g_status w4a8_gemm_workspace_size(int64_t L, int64_t M, int64_t N, int64_t K, int64_t splits,
                                     size_t *bytes);
fp4g_status nv_fp4_gemm_split(int64_t L, int64_t M, int64_t N, int64_t K,
                              const void *A, const void *sfA, float global_a,
                              const void *B, const void *sfB, float global_b,
                              void *D, int d_type, int64_t splits,
                              void *workspace, size_t workspace_bytes, void *stream);
fp4g_status w4a8_gemm_split(int64_t L, int64_t M, int64_t N, int64_t K,
                            const void *A, const float *sa,
                            const void *B, const void *sB,
                            void *D, int d_type, int64_t splits,
                            void *workspace, size_t workspace_bytes, void *stream);
fp4g_status w4a8_gemm_prepacked_split(int64_t M, int64_t N, int64_t K,
                                      const void *A, const float *sa,
                                      const void *Bp, const void *Sp,
                                      void *D, int d_type, int64_t splits,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Pre-packed decode weights (a load-time step, like the weight re-encoding and
 * re-ordering that the Hopper CUTLASS/CuTe DSL blog post describes for W4A8 in
 * section "The W4A8 kernel: the same four definitions, with the operands
 * swapped").  The MXFP4 weight operand of fp4_gemv, B [N][K/2] and sfB [N][K/32],
 * is re-ordered into the register layout of the 16x16x128 FP4 matrix
 * instruction, with G = ceil(N/16) groups of 16 rows, KT = K/128 steps,
 * KC = ceil(KT/4), and lane l = 16*slot + r (slot 0..3, r 0..15):
 *   Bp bytes [G][KT][64 lanes][16]:  Bp[g][s][l][b] = B[16g+r][64s + 16*slot + b]
 *   Sp dwords [G][KC][64 lanes]:     byte i of Sp[g][c][l] = sfB[16g+r][4(4c+i) + slot]
 * Rows past N are zero codes with scale 127; steps past KT in the last chunk have
 * scale 127.
 *
 * fp4_gemv_prepack_size: bytes of Bp (G*KT*1024) and Sp (G*KC*256); neither
 *   pointer may be NULL.  Sizes as for fp4_gemv (K % 128 == 0).
 * fp4_gemv_prepack: writes Bp and Sp from B and sfB on `stream`.  B 16-byte
 *   aligned, sfB any alignment; Bp 16-byte and Sp 4-byte aligned, of the sizes
 *   above; outputs must not overlap each other or the inputs.  N == 0 or K == 0
 *   is a no-op.
 * fp4_gemv_prepacked: fp4_gemv (1 <= M <= 16 tokens, same A, sfA and D layouts
 *   and result) with the weights given as Bp and Sp.  Bp 16-byte and Sp 4-byte
 *   aligned; D must not overlap any input.  M > 16 returns FP4G_EUNSUPPORTED.
 *   Measured on MI355X with cold weights it is the faster of the two at K >= 8192
 *   (row pitches of 4 KB and more), and fp4_gemv at K <= 4096. */
fp4g_status fp4_gemv_prepack_size(int64_t N, int64_t K, size_t *weight_bytes, size_t *scale_bytes);
fp4g_status fp4_gemv_prepack(int64_t N, int64_t K, const void *B, const void *sfB,
                             void *Bp, void *Sp, void *stream);
fp4g_status fp4_gemv_prepacked(int64_t M, int64_t N, int64_t K,
                               const void *A, const void *sfA,
                               const void *Bp, const void *Sp,
                               void *D, int d_type, void *stream);

/* MX quantizer: X[rows][K] (fp32 or bf16 by x_type) -> E2M1 codes [rows][K/2] (low
 * nibble = even k, the operand layout above) and E8M0 scales [rows][K/32].  It makes
 * the activation operand of mx_fp4_gemm and fp4_gemv from activations, the
 * inference setting of the issue page ("Impact") and of the cute-rs page's MXFP4
 * GEMV ("Where to Go Next").  The pages fix no rounding rule; the rule is max-abs
 * per 32-element block:
 *   e = clamp(floor(log2 max|x|) - 2 + 127, 0, 254)   (127 for an all-zero block),
 *   code = the E2M1 value nearest to x * 2^(127 - e), ties to the even mantissa bit,
 *          magnitudes past 6 saturating to 6; a zero result is +0;
 *   a block holding an infinity or NaN gets scale 0xFF (NaN) and zero codes.
 * Requires rows*K <= 2^50 (FP4G_EINVAL otherwise) and K a multiple of 32
 * (FP4G_EUNSUPPORTED otherwise); X and codes 16-byte
 * aligned; the three buffers must not overlap.  rows == 0 or K == 0 is a no-op. */
fp4g_status mx_fp4_quantize(int64_t rows, int64_t K, const void *X, int x_type,
                            void *codes, void *scales, void *stream);

/* NV quantizer: X[rows][K] (fp32 or bf16 by x_type) and an fp32 global scale g ->
 * E2M1 codes [rows][K/2] (low nibble = even k) and E4M3 scales [rows][K/16], the
 * operand of nv_fp4_gemm with global scale g (16-element E4M3 blocks: the issue
 * page's "Scale Factor Granularity").  The pages fix no rounding rule; the rule is
 * max-abs per 16-element block, every step in IEEE fp32:
 *   sv = max|x| / (6 * g)   (6 * g first, then the division),
 *   s  = the E4M3 code nearest to sv, ties to the even code, values past 448
 *        saturating to 448 (0x7E),
 *   code = the E2M1 value nearest to x * inv, with inv = min(1 / (e4m3(s) * g),
 *          FLT_MAX) (one reciprocal per block), ties to the even mantissa bit,
 *          magnitudes past 6 saturating to 6; a zero result is +0;
 *   a scale that decodes to 0 gives all-zero codes; a block holding an infinity or
 *   NaN gets scale 0x7F (NaN) and zero codes.
 * The caller chooses g (for example max|X| / (448 * 6), which puts the largest block
 * scale near the top of the E4M3 range); it must be finite and positive
 * (FP4G_EINVAL otherwise).  Requires rows*K <= 2^50 (FP4G_EINVAL) and K a multiple
 * of 16 (FP4G_EUNSUPPORTED); X 16-byte and codes 8-byte aligned; the three buffers
 * must not overlap.  rows == 0 or K == 0 is a no-op. */
fp4g_status nv_fp4_quantize(int64_t rows, int64_t K, const void *X, int x_type, float global_scale,
                            void *codes, void *scales, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *fp4g_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP4GEMM_H */
