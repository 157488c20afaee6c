/*
 * oracle.c -- plain, slow, fp64 CPU reference for the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library: every decoder below is
 * written from the bit-field definitions of the formats.
 *
 * What it computes (block-scaled contraction):
 *   D[m][n] = sum_k (a[m][k] * sfa[m][k/V]) * (b[n][k] * sfb[n][k/V])
 * with a, b E2M1 codes and one scale per V consecutive K elements:
 *   - MXFP4: V = 32, E8M0 scales (page 3, "Block-Scaled MXFP4 GEMM in cute-rs
 *     (SM120a)": Float8E8M0FNU scales, one scale pair per K=64 step).
 *   - NVFP4: V = 16, E4M3 scales (page 1, "Scale Factor Granularity" and the
 *     "Code Reference" block: sf_dtype Float8E4M3FN, sf_vec_size 16), followed
 *     by one fp32 global scale per operand.
 *   - W4A8: FP8 E4M3 activations times signed INT4 weights with one scale per
 *     weight row per 128-element K tile (page 2, "The W4A8 kernel: the same
 *     four definitions, with the operands swapped": TileShapeK = 128; and
 *     "What changes in the W4A8 builder", item 4: one scale per row per K
 *     tile), and one fp32 scale per activation row.
 *
 * Every product and sum is taken in fp64, in increasing k, with no blocking.
 * Besides D, each routine returns S[m][n] = sum_k |a_hat * b_hat| (all scales
 * folded in), the magnitude that the parity tolerance is relative to.
 *
 * Layouts (the plainest reading; the pages do not fix them):
 *   FP4 / INT4 operand X[rows][K/2] bytes, row-major, K contiguous; the low
 *   nibble of byte j holds element 2j, the high nibble element 2j+1.
 *   Scales sf[rows][K/V] bytes, row-major.  FP8 operand A[M][K] bytes.
 *   W4A8 group scales sB[N][K/128] as raw bf16 bit patterns.  D[M][N] fp64.
 *
 * Return value: 0 on success, -1 on an argument error (K not a multiple of V
 * or of 2, null pointer, negative size).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ---- scalar decoders, each from its format's bit fields ---------------- */

/* E2M1 ("Float4E2M1FN", page 1 "What Works"): 1 sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; exponent field 0 is subnormal (0.5 * m); no
 * infinities or NaNs ("FN"). */
double oracle_e2m1(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0 ("Float8E8M0FNU", page 3 section 1): unsigned power of two, value
 * 2^(e-127); the all-ones code is NaN, there are no zeros or infinities. */
double oracle_e8m0(unsigned e) {
    e &= 0xFFu;
    if (e == 0xFFu) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* E4M3 with the "FN" convention ("Float8E4M3FN", page 1 "Code Reference"):
 * 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
 * subnormal; exponent 15 with mantissa 7 is NaN; no infinities; max 448. */
double oracle_e4m3fn(unsigned b) {
    b &= 0xFFu;
    unsigned s = b >> 7, E = (b >> 3) & 15u, M = b & 7u;
    double mag;
    if (E == 15u && M == 7u) return NAN;
    if (E == 0u) mag = ldexp((double)M / 8.0, -6);
    else mag = ldexp(1.0 + (double)M / 8.0, (int)E - 7);
    return s ? -mag : mag;
}

/* Signed INT4 ("int4b_t", page 2): two's complement nibble, -8..7. */
int oracle_int4(unsigned n) {
    n &= 0xFu;
    return (n < 8u) ? (int)n : (int)n - 16;
}

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16(uint16_t u) {
    uint32_t bits = (uint32_t)u << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Nibble k of a packed row: low nibble = even k. */
static unsigned nibble(const uint8_t *row, int64_t k) {
    uint8_t byte = row[k >> 1];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 0xFu);
}

/* ---- one output element of each product ------------------------------------
 *
 * Each routine below computes one D[m][n] and its S[m][n] from the operand rows it
 * is given.  The full products and the sampled entry point both call them, so every
 * product is written out once. */

typedef double (*scale_fn)(unsigned);

/* Block-scaled FP4: sum_k (e2m1(a_k) * scale(sfa[k/V])) * (e2m1(b_k) * scale(sfb[k/V])). */
static void fp4_dot(int64_t K, int64_t V, scale_fn dec_scale,
                    const uint8_t *arow, const uint8_t *sfarow,
                    const uint8_t *brow, const uint8_t *sfbrow,
                    double *d, double *s) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a_hat = oracle_e2m1(nibble(arow, k)) * dec_scale(sfarow[k / V]);
        double b_hat = oracle_e2m1(nibble(brow, k)) * dec_scale(sfbrow[k / V]);
        double p = a_hat * b_hat;
        acc += p;
        mag += fabs(p);
    }
    *d = acc;
    *s = mag;
}

/* MXFP4: V = 32, E8M0 scales. */
static void mx_dot(int64_t K, const uint8_t *arow, const uint8_t *sfarow,
                   const uint8_t *brow, const uint8_t *sfbrow, double *d, double *s) {
    fp4_dot(K, 32, oracle_e8m0, arow, sfarow, brow, sfbrow, d, s);
}

/* NVFP4: V = 16, E4M3 scales, then the product of the two fp32 global scales
 * (exact in fp64: two 24-bit significands) multiplies D, and its magnitude S. */
static void nv_dot(int64_t K, const uint8_t *arow, const uint8_t *sfarow, double gA,
                   const uint8_t *brow, const uint8_t *sfbrow, double gB, double *d, double *s) {
    double dd, ss;
    fp4_dot(K, 16, oracle_e4m3fn, arow, sfarow, brow, sfbrow, &dd, &ss);
    const double g = gA * gB;
    *d = dd * g;
    *s = ss * fabs(g);
}

/* W4A8: sa * sum_g bf16(sB[g]) * sum_{k in group g} e4m3(a_k) * int4(b_k), groups of
 * 128 consecutive K elements.  S is the same sum with every factor in absolute value. */
#define W4A8_GROUP 128
static void w4a8_dot(int64_t K, const uint8_t *arow, double row_scale,
                     const uint8_t *brow, const uint16_t *sbrow, double *d, double *s) {
    double acc = 0.0, mag = 0.0;
    for (int64_t g = 0; g < K / W4A8_GROUP; ++g) {
        double w4_part = 0.0, w4_part_mag = 0.0;
        for (int64_t k = g * W4A8_GROUP; k < (g + 1) * W4A8_GROUP; ++k) {
            double p = oracle_e4m3fn(arow[k]) * (double)oracle_int4(nibble(brow, k));
            w4_part += p;
            w4_part_mag += fabs(p);
        }
        double gs = oracle_bf16(sbrow[g]);
        acc += gs * w4_part;
        mag += fabs(gs) * w4_part_mag;
    }
    *d = row_scale * acc;
    *s = fabs(row_scale) * mag;
}

/* FP8 blockwise: sum_g sA[g] * sB[g] * sum_{k in group g} e4m3(a_k) * e4m3(b_k), groups
 * of 128 consecutive K elements, one fp32 scale per row per group. */
#define FP8_BLOCK 128
static void fp8b_dot(int64_t K, const uint8_t *arow, const float *sarow,
                     const uint8_t *brow, const float *sbrow, double *d, double *s) {
    double acc = 0.0, mag = 0.0;
    for (int64_t g = 0; g < K / FP8_BLOCK; ++g) {
        double fp8_part = 0.0, fp8_part_mag = 0.0;
        for (int64_t k = g * FP8_BLOCK; k < (g + 1) * FP8_BLOCK; ++k) {
            double p = oracle_e4m3fn(arow[k]) * oracle_e4m3fn(brow[k]);
            fp8_part += p;
            fp8_part_mag += fabs(p);
        }
        const double sc = (double)sarow[g] * (double)sbrow[g];
        acc += sc * fp8_part;
        mag += fabs(sc) * fp8_part_mag;
    }
    *d = acc;
    *s = mag;
}

/* ---- full products (rows [row0, row1) of D and S, written to D[0 .. (row1-row0)*N)) -- */

static int check_rows(int64_t M, int64_t N, int64_t K, int64_t kdiv, const void *A, const void *sfA,
                      const void *B, const void *sfB, int64_t row0, int64_t row1, double *D, double *S) {
    if (M < 0 || N < 0 || K < 0 || (K % kdiv) != 0) return -1;
    if (row0 < 0 || row1 > M || row0 > row1) return -1;
    if ((M && N && K) && (!A || !sfA || !B || !sfB)) return -1;
    if ((row1 > row0 && N) && (!D || !S)) return -1;
    return 0;
}

/* MXFP4: V = 32, E8M0 scales.  The M <= 16 GEMV is the same operation. */
int oracle_mx_gemm_rows(int64_t M, int64_t N, int64_t K,
                        const uint8_t *A, const uint8_t *sfA,
                        const uint8_t *B, const uint8_t *sfB,
                        int64_t row0, int64_t row1, double *D, double *S) {
    if (check_rows(M, N, K, 32, A, sfA, B, sfB, row0, row1, D, S)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = row0; m < row1; ++m)
        for (int64_t n = 0; n < N; ++n)
            mx_dot(K, A + m * (K / 2), sfA + m * (K / 32), B + n * (K / 2), sfB + n * (K / 32),
                   &D[(m - row0) * N + n], &S[(m - row0) * N + n]);
    return 0;
}

int oracle_mx_gemm(int64_t M, int64_t N, int64_t K,
                   const uint8_t *A, const uint8_t *sfA,
                   const uint8_t *B, const uint8_t *sfB, double *D, double *S) {
    return oracle_mx_gemm_rows(M, N, K, A, sfA, B, sfB, 0, M, D, S);
}

/* NVFP4: V = 16, E4M3 scales, then D *= gA * gB and S *= |gA * gB|. */
int oracle_nv_gemm_rows(int64_t M, int64_t N, int64_t K,
                        const uint8_t *A, const uint8_t *sfA, double gA,
                        const uint8_t *B, const uint8_t *sfB, double gB,
                        int64_t row0, int64_t row1, double *D, double *S) {
    if (check_rows(M, N, K, 16, A, sfA, B, sfB, row0, row1, D, S)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = row0; m < row1; ++m)
        for (int64_t n = 0; n < N; ++n)
            nv_dot(K, A + m * (K / 2), sfA + m * (K / 16), gA, B + n * (K / 2), sfB + n * (K / 16), gB,
                   &D[(m - row0) * N + n], &S[(m - row0) * N + n]);
    return 0;
}

int oracle_nv_gemm(int64_t M, int64_t N, int64_t K,
                   const uint8_t *A, const uint8_t *sfA, double gA,
                   const uint8_t *B, const uint8_t *sfB, double gB, double *D, double *S) {
    return oracle_nv_gemm_rows(M, N, K, A, sfA, gA, B, sfB, gB, 0, M, D, S);
}

/* W4A8: A [M][K] E4M3 codes, sa [M] fp32, B [N][K/2] INT4, sB [N][K/128] bf16 bits. */
int oracle_w4a8_gemm_rows(int64_t M, int64_t N, int64_t K,
                          const uint8_t *A, const float *sa,
                          const uint8_t *B, const uint16_t *sB,
                          int64_t row0, int64_t row1, double *D, double *S) {
    if (check_rows(M, N, K, W4A8_GROUP, A, sa, B, sB, row0, row1, D, S)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = row0; m < row1; ++m)
        for (int64_t n = 0; n < N; ++n)
            w4a8_dot(K, A + m * K, (double)sa[m], B + n * (K / 2), sB + n * (K / W4A8_GROUP),
                     &D[(m - row0) * N + n], &S[(m - row0) * N + n]);
    return 0;
}

int oracle_w4a8_gemm(int64_t M, int64_t N, int64_t K,
                     const uint8_t *A, const float *sa,
                     const uint8_t *B, const uint16_t *sB, double *D, double *S) {
    return oracle_w4a8_gemm_rows(M, N, K, A, sa, B, sB, 0, M, D, S);
}

/* FP8 blockwise-scaled GEMM.  The issue page ("What Works", "Background" and
 * "Scale Factor Granularity") names the FP8 blockwise GEMM as the existing
 * Blackwell example that the FP4 kernels extend, with a scale granularity of 128
 * along K.  The plainest reading of that granularity: each row of each operand
 * carries one fp32 scale per 128 consecutive K elements, and
 *   D[m][n] = sum_g sA[m][g] * sB[n][g] * sum_{k in group g} e4m3(A[m][k]) * e4m3(B[n][k]).
 * A [M][K] and B [N][K] are E4M3 codes (K-major), sA [M][K/128], sB [N][K/128]. */
int oracle_fp8b_gemm_rows(int64_t M, int64_t N, int64_t K,
                          const uint8_t *A, const float *sA,
                          const uint8_t *B, const float *sB,
                          int64_t row0, int64_t row1, double *D, double *S) {
    if (check_rows(M, N, K, FP8_BLOCK, A, sA, B, sB, row0, row1, D, S)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = row0; m < row1; ++m)
        for (int64_t n = 0; n < N; ++n)
            fp8b_dot(K, A + m * K, sA + m * (K / FP8_BLOCK), B + n * K, sB + n * (K / FP8_BLOCK),
                     &D[(m - row0) * N + n], &S[(m - row0) * N + n]);
    return 0;
}

/* Sampled outputs: the same definitions evaluated only at the listed (m, n)
 * pairs, for shapes whose full product is too slow on the CPU.  kind selects
 * the operation: 0 = MXFP4, 1 = NVFP4 (gA, gB used), 2 = W4A8 (A is FP8,
 * sfA is the fp32 row-scale array, sfB the bf16 group scales), 3 = FP8 blockwise
 * (A and B are FP8, sfA and sfB their fp32 group scales). */
int oracle_sampled(int kind, int64_t M, int64_t N, int64_t K,
                   const void *A, const void *sfA, double gA,
                   const void *B, const void *sfB, double gB,
                   const int64_t *ms, const int64_t *ns, int64_t count,
                   double *D, double *S) {
    if (count < 0 || (count && (!ms || !ns || !D || !S))) return -1;
    if (kind < 0 || kind > 3 || K < 0) return -1;
    const int64_t kdiv = kind == 0 ? 32 : kind == 1 ? 16 : 128;
    if (K % kdiv) return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
    const uint8_t *a8 = (const uint8_t *)A, *b8 = (const uint8_t *)B;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = ms[i], n = ns[i];
        if (kind == 0)
            mx_dot(K, a8 + m * (K / 2), (const uint8_t *)sfA + m * (K / 32), b8 + n * (K / 2),
                   (const uint8_t *)sfB + n * (K / 32), &D[i], &S[i]);
        else if (kind == 1)
            nv_dot(K, a8 + m * (K / 2), (const uint8_t *)sfA + m * (K / 16), gA, b8 + n * (K / 2),
                   (const uint8_t *)sfB + n * (K / 16), gB, &D[i], &S[i]);
        else if (kind == 2)
            w4a8_dot(K, a8 + m * K, (double)((const float *)sfA)[m], b8 + n * (K / 2),
                     (const uint16_t *)sfB + n * (K / W4A8_GROUP), &D[i], &S[i]);
        else
            fp8b_dot(K, a8 + m * K, (const float *)sfA + m * (K / FP8_BLOCK), b8 + n * K,
                     (const float *)sfB + n * (K / FP8_BLOCK), &D[i], &S[i]);
    }
    return 0;
}

/* ---- truncation bound of the FP8 matrix instruction ----------------------
 *
 * Not a product: a term of the comparison rule for the contractions that run on
 * gfx950's scaled FP8 matrix instruction (W4A8 and FP8 blockwise).  Measured on the
 * GPU, that instruction truncates the products of each aligned run of 8 consecutive K
 * elements toward zero to a multiple of 2^(E - 13), E the largest exponent sum
 * e(a) + e(b) in the run (e = the unbiased exponent field of the E4M3 code, -6 for
 * subnormals), before adding them.  Each product therefore loses exactly |a b| mod
 * 2^(E - 13); H sums those magnitudes over every run with the scales folded in, which
 * bounds the error of the sum.
 * W4A8 weights enter either as one E4M3 value q (split = 0) or as the two exact parts
 * v = q mod 8 and -8 [q < 0], each its own instruction, with v as the E4M3 value v
 * (split = 1) or as the subnormal code v, worth v * 2^-9, scaled by 2^9 in the
 * instruction (split = 2): its exponent field is then -6 + 9 = 3 whatever v is. */
static int e4m3_exp_field(unsigned c) {
    const unsigned E = (c >> 3) & 15u;
    return E == 0 ? -6 : (int)E - 7;
}

/* exponent field of the integer magnitude u = 1..8 as an E4M3 value */
static int int_exp_field(int u) { return u >= 8 ? 3 : u >= 4 ? 2 : u >= 2 ? 1 : 0; }

/* loss of one run: products p[i] with exponent sums e[i] (valid where p[i] != 0) */
static double run_loss(const double *p, const int *e, int n) {
    int E = -100000;
    for (int i = 0; i < n; ++i)
        if (p[i] != 0.0 && e[i] > E) E = e[i];
    if (E == -100000) return 0.0;
    const double unit = ldexp(1.0, E - 13);
    double loss = 0.0;
    for (int i = 0; i < n; ++i) loss += fmod(p[i], unit);    /* what truncation drops; fmod is exact */
    return loss;
}

static double fp8_bound_one(int kind, int split, int64_t K, const uint8_t *arow, const void *sa_row,
                            const uint8_t *brow, const void *sb_row, double row_scale) {
    double H = 0.0;
    for (int64_t g = 0; g < K / 128; ++g) {
        double group = 0.0;
        for (int64_t r = g * 128; r < (g + 1) * 128; r += 8) {
            double p1[8], p2[8];
            int e1[8], e2[8];
            for (int i = 0; i < 8; ++i) {
                const int64_t k = r + i;
                const double am = fabs(oracle_e4m3fn(arow[k]));
                const int ea = e4m3_exp_field(arow[k]);
                if (kind == 3) {
                    p1[i] = am * fabs(oracle_e4m3fn(brow[k]));
                    e1[i] = ea + e4m3_exp_field(brow[k]);
                    p2[i] = 0.0;
                    e2[i] = 0;
                } else if (split) {
                    const int q = oracle_int4(nibble(brow, k));
                    const int v = q & 7, neg = q < 0;
                    p1[i] = am * v;
                    e1[i] = split == 2 ? ea + 3 : ea + int_exp_field(v);
                    p2[i] = neg ? 8.0 * am : 0.0;
                    e2[i] = ea + 3;
                } else {
                    const int q = oracle_int4(nibble(brow, k));
                    const int u = q < 0 ? -q : q;
                    p1[i] = am * u;
                    e1[i] = ea + int_exp_field(u);
                    p2[i] = 0.0;
                    e2[i] = 0;
                }
            }
            group += run_loss(p1, e1, 8) + run_loss(p2, e2, 8);
        }
        if (kind == 3)
            H += fabs((double)((const float *)sa_row)[g] * (double)((const float *)sb_row)[g]) * group;
        else
            H += fabs(oracle_bf16(((const uint16_t *)sb_row)[g])) * group;
    }
    return kind == 3 ? H : fabs(row_scale) * H;
}

/* kind 2 = W4A8 (sfA: fp32 row scales [M], sfB: bf16 group scales [N][K/128]),
 * kind 3 = FP8 blockwise (sfA [M][K/128], sfB [N][K/128] fp32).  H for rows
 * [row0, row1) into H[0 .. (row1-row0)*N), or, when ms is not NULL, for the count pairs
 * (ms[i], ns[i]) into H[0 .. count). */
int oracle_fp8_bound(int kind, int split, int64_t M, int64_t N, int64_t K,
                     const uint8_t *A, const void *sfA, const uint8_t *B, const void *sfB,
                     int64_t row0, int64_t row1, const int64_t *ms, const int64_t *ns, int64_t count,
                     double *H) {
    if ((kind != 2 && kind != 3) || split < 0 || split > 2 || M < 0 || N < 0 || K < 0 || K % 128 || !H)
        return -1;
    const int64_t b_ld = kind == 3 ? K : K / 2;
    if (ms) {
        for (int64_t i = 0; i < count; ++i)
            if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t i = 0; i < count; ++i) {
            const int64_t m = ms[i], n = ns[i];
            H[i] = kind == 3
                ? fp8_bound_one(3, 0, K, A + m * K, (const float *)sfA + m * (K / 128), B + n * b_ld,
                                (const float *)sfB + n * (K / 128), 1.0)
                : fp8_bound_one(2, split, K, A + m * K, NULL, B + n * b_ld,
                                (const uint16_t *)sfB + n * (K / 128), (double)((const float *)sfA)[m]);
        }
        return 0;
    }
    if (row0 < 0 || row1 > M || row0 > row1) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = row0; m < row1; ++m)
        for (int64_t n = 0; n < N; ++n)
            H[(m - row0) * N + n] = kind == 3
                ? fp8_bound_one(3, 0, K, A + m * K, (const float *)sfA + m * (K / 128), B + n * b_ld,
                                (const float *)sfB + n * (K / 128), 1.0)
                : fp8_bound_one(2, split, K, A + m * K, NULL, B + n * b_ld,
                                (const uint16_t *)sfB + n * (K / 128), (double)((const float *)sfA)[m]);
    return 0;
}

/* ---- MX quantizer: fp32 -> E2M1 codes + E8M0 block scales ---------------
 *
 * The step before the GEMM for activations: the issue page's "Impact" section
 * places FP4 GEMMs in inference, and the cute-rs page's "Where to Go Next"
 * table lists the MXFP4 GEMV, whose activations must arrive as E2M1 codes
 * with E8M0 scales.  The pages fix no rounding rule; the reading taken is the
 * max-abs rule, per block of 32 consecutive K elements with amax = max |x|:
 *   e = clamp(floor(log2 amax) - 2 + 127, 0, 254)     (e = 127 for amax = 0)
 * so the block's largest magnitude lands in [4, 8) once scaled by 2^(127-e);
 * each element becomes x * 2^(127-e) rounded to the NEAREST E2M1 value, a
 * tie going to the code whose mantissa bit is 0, so magnitudes past 6
 * saturate to 6.  A result of magnitude 0 is encoded +0 (code 0).  A block
 * holding an infinity or a NaN gets the NaN scale 0xFF and all-zero codes.
 * The nearest value is found by trying all eight magnitudes through
 * oracle_e2m1, the decoder written from the format's bit fields.
 *
 * x [rows][K] fp32, codes [rows][K/2] (low nibble = even k), scales
 * [rows][K/32].  Returns 0, or -1 on bad arguments (K not a multiple of 32). */
static unsigned e2m1_nearest_magnitude(double y) {
    /* saturation first: far above 6 every distance rounds to the same double */
    if (y >= 6.0) return 7;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        const double d = fabs(y - oracle_e2m1(c));
        if (d < best_d || (d == best_d && (c & 1u) == 0 && (best & 1u) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

int oracle_mx_quantize(int64_t rows, int64_t K, const float *x, uint8_t *codes, uint8_t *scales) {
    if (rows < 0 || K < 0 || K % 32) return -1;
    if (rows && K && (!x || !codes || !scales)) return -1;
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *blk = x + r * K + 32 * b;
            uint8_t *out = codes + r * (K / 2) + 16 * b;
            int finite = 1;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                if (!isfinite(blk[i])) finite = 0;
                else if (fabs((double)blk[i]) > amax) amax = fabs((double)blk[i]);
            }
            if (!finite) {
                scales[r * nb + b] = 0xFF;
                memset(out, 0, 16);
                continue;
            }
            int e = 127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1 */
                e = ex - 1 - 2 + 127;
                if (e < 0) e = 0;
                if (e > 254) e = 254;
            }
            scales[r * nb + b] = (uint8_t)e;
            for (int i = 0; i < 32; i += 2) {
                unsigned nib[2];
                for (int h = 0; h < 2; ++h) {
                    const double y = ldexp((double)blk[i + h], 127 - e);
                    unsigned c = e2m1_nearest_magnitude(fabs(y));
                    if (c != 0 && y < 0.0) c |= 8u;
                    nib[h] = c;
                }
                out[i / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
    }
    return 0;
}

/* ---- NV quantizer (NVFP4 operand from activations) ---------------------
 *
 * The NVFP4 counterpart of oracle_mx_quantize: E2M1 codes with one E4M3 scale
 * per 16 consecutive K elements (the issue page's "Scale Factor Granularity":
 * sf_vec_size 16 with Float8E4M3FN scales) and one fp32 global scale g per
 * tensor, supplied by the caller.  The pages fix no rounding rule; the reading
 * taken is max-abs with round-to-nearest on exact real quotients, per block with
 * amax = max |x|:
 *   s = the E4M3 code nearest to amax / (6 g), a tie going to the even code,
 *       values past 448 saturating to 448 (code 0x7E);
 *   if s decodes to 0 every code is +0; otherwise each element becomes the E2M1
 *       value nearest to x / (e4m3(s) g), a tie going to the even mantissa bit,
 *       magnitudes past 6 saturating to 6, a zero result encoded +0.
 * A block holding an infinity or NaN gets the NaN scale 0x7F and zero codes.
 *
 * Both quotients are taken in fp64, and that decides every code exactly.  The
 * operands are fp32 (24-bit significands), e4m3(s) has 4 significant bits and 6
 * has 2, so 6 g and e4m3(s) g are exact in fp64.  A rounding boundary of the
 * grid (an E4M3 midpoint, 5 bits, or an E2M1 midpoint, 3 bits) times the divisor
 * has at most 31 significant bits; amax or x differs from it by zero or by at
 * least 2^-32 of its size, while the fp64 quotient is off by at most 2^-53 of its
 * size.  So the fp64 quotient lies on the same side of every boundary as the
 * exact one, and equals a boundary exactly when the exact quotient does.  The
 * nearest value is then found by trying every candidate (differences of
 * neighbouring grid values from a quotient between them are exact in fp64).
 *
 * x [rows][K] fp32, codes [rows][K/2], scales [rows][K/16].  Returns 0, or -1 on
 * bad arguments (K not a multiple of 16, g not finite and positive). */
static unsigned e4m3_nearest_code(double sv) {
    /* saturation first: far above 448 every distance rounds to the same double */
    if (sv >= 448.0) return 0x7E;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c <= 0x7E; ++c) {
        const double d = fabs(sv - oracle_e4m3fn(c));
        if (d < best_d || (d == best_d && !(c & 1u) && (best & 1u))) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

int oracle_nv_quantize(int64_t rows, int64_t K, const float *x, float g, uint8_t *codes, uint8_t *scales) {
    if (rows < 0 || K < 0 || K % 16 || !(g > 0.0f) || !isfinite(g)) return -1;
    if (rows && K && (!x || !codes || !scales)) return -1;
    const int64_t nb = K / 16;
    const double gd = (double)g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *blk = x + r * K + 16 * b;
            uint8_t *out = codes + r * (K / 2) + 8 * b;
            int finite = 1;
            double amax = 0.0;
            for (int i = 0; i < 16; ++i) {
                if (!isfinite(blk[i])) {
                    finite = 0;
                    continue;
                }
                if (fabs((double)blk[i]) > amax) amax = fabs((double)blk[i]);
            }
            if (!finite) {
                scales[r * nb + b] = 0x7F;
                memset(out, 0, 8);
                continue;
            }
            const unsigned s = e4m3_nearest_code(amax / (6.0 * gd));
            scales[r * nb + b] = (uint8_t)s;
            const double divisor = oracle_e4m3fn(s) * gd;
            if (divisor == 0.0) {
                memset(out, 0, 8);
                continue;
            }
            for (int i = 0; i < 16; i += 2) {
                unsigned nib[2];
                for (int h = 0; h < 2; ++h) {
                    const double q = (double)blk[i + h] / divisor;
                    unsigned c = e2m1_nearest_magnitude(fabs(q));
                    if (c != 0 && q < 0.0) c |= 8u;
                    nib[h] = c;
                }
                out[i >> 1] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
        }
    }
    return 0;
}
