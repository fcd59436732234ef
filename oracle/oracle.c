/*
 * oracle.c -- plain CPU reference for the fine-grained block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle that the GPU path is
 * checked against. It shares no code, header, table or helper with the GPU
 * library, and only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it. Nothing in the product path calls it.
 *
 * What it computes (written from the pages, in their notation):
 *
 *   D[m, n] = bf16_rne( sum_kb  (sA[m, kb] * sB[n/128, kb])
 *                               * sum_{k in block kb} dec(A[m, k]) * dec(B[n, k]) )
 *
 *  - The scaled product is taken per 128-wide K block and added to a wider
 *    accumulator; the scale product changes with kb, so it cannot be pulled
 *    out of the K loop (lpnh.cn DeepGEMM article, §2.3; hotdry.top
 *    fine-grained scaling article, "two-level accumulation").
 *  - LHS scales are per 1x128 tile, RHS scales per 128x128 tile (hotdry.top,
 *    "fine-grained scaling core design").
 *  - dec() is the e4m3 code: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 *    largest finite magnitude 448 (rkmt.cn walkthrough §2.1 and §5.2; lpnh.cn
 *    §2.1); code S.1111.111 is NaN and there is no infinity.
 *  - Output is bf16, rounded once, to nearest with ties to even.
 *
 * Precision. Every decoded e4m3 value is a multiple of 2^-9 below 2^9, so a
 * product is a multiple of 2^-18 below 2^18 and any sum of at most 128 such
 * products is an integer multiple of 2^-18 below 2^43: it is exact in binary64
 * whatever the order. The per-block scale product (24 x 24 significant bits)
 * is exact in binary64 as well. The only roundings are the fp64 additions
 * across K blocks (relative 2^-53 each) and the single final bf16 rounding.
 *
 * Grouped variants apply the same element formula per row:
 *  - contiguous: row r uses expert ids[r] if 0 <= ids[r] < G; any other id
 *    marks a row that is not produced (its output is left untouched);
 *  - masked: group g produces rows m < clamp(masked_m[g], 0, M_max); the other
 *    rows are left untouched.
 *
 * Parity pins: every function below is pinned by the "not gpu" tests against
 * closed forms, hand-worked cases, brute-force fp64 matmul of the dequantised
 * inputs, an exact int64 matmul of the integer codes, and torch's CPU casts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define BLK 128

/* e4m3 decode, from the bit fields (sign s, exponent e, mantissa f). */
double dgo_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int f = code & 7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -9);            /* subnormal: f * 2^-6 / 8 */
    else
        mag = ldexp((double)(8 + f), e - 10);  /* (1 + f/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Single round-to-nearest-even from binary64 to bfloat16 (returns the bits).
 * bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
uint16_t dgo_bf16_rne(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);               /* a = m * 2^ex, 0.5 <= m < 1 */
    int E = ex - 1;              /* floor(log2 a) */
    if (E < -126)
        E = -126;                /* subnormal range: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, E - 7);
    double r = rint(a / quantum) * quantum;  /* a/quantum is exact; rint is ties-to-even */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80;    /* overflow to infinity */
    if (r < ldexp(1.0, -126))    /* subnormal (or rounds up to min normal: field 128 -> exp 1) */
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    frexp(r, &ex);
    E = ex - 1;
    uint16_t mant = (uint16_t)(r / ldexp(1.0, E - 7) - 128.0);
    return sign | (uint16_t)((E + 127) << 7) | mant;
}

static double dec_table[256];
static int dec_ready = 0;

static void init_table(void)
{
    if (dec_ready)
        return;
    for (int c = 0; c < 256; ++c)
        dec_table[c] = dgo_e4m3_decode((uint8_t)c);
    dec_ready = 1;
}

/* Exact sum of the 128 products of one K block. */
double dgo_block_partial(const uint8_t *a, const uint8_t *b)
{
    init_table();
    double p = 0.0;
    for (int k = 0; k < BLK; ++k)
        p += dec_table[a[k]] * dec_table[b[k]];
    return p;
}

/* One output element before rounding:
 *   sum_kb (sa[kb] * sb[kb]) * sum_{k in kb} dec(a[k]) dec(b[k]). */
static double element(const uint8_t *a, const float *sa, int64_t sa_kb,
                      const uint8_t *b, const float *sb, int64_t sb_kb, int64_t K)
{
    double acc = 0.0;
    for (int64_t kb = 0; kb < K / BLK; ++kb) {
        double partial = 0.0;
        for (int64_t k = kb * BLK; k < (kb + 1) * BLK; ++k)
            partial += dec_table[a[k]] * dec_table[b[k]];
        double scale = (double)sa[kb * sa_kb] * (double)sb[kb * sb_kb];
        acc += partial * scale;
    }
    return acc;
}

static void set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

int dgo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Dense NT: D[M,N] from A[M,K] (row stride lda), B[N,K] (row stride ldb),
 * sA[m,kb] at sA[m*sa_m + kb*sa_kb], sB[nb,kb] at sB[nb*sb_nb + kb*sb_kb].
 * acc (optional, [M*N] row-major) receives the fp64 values, D the bf16 bits. */
void dgo_gemm_nt(const uint8_t *A, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                 const uint8_t *B, int64_t ldb, const float *sB, int64_t sb_nb, int64_t sb_kb,
                 int64_t M, int64_t N, int64_t K,
                 double *acc, uint16_t *D, int64_t ldd, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = element(A + m * lda, sA + m * sa_m, sa_kb,
                               B + n * ldb, sB + (n / BLK) * sb_nb, sb_kb, K);
            if (acc)
                acc[m * N + n] = v;
            D[m * ldd + n] = dgo_bf16_rne(v);
        }
}

/* Dense NT at chosen output points (ms[i], ns[i]). */
void dgo_gemm_nt_points(const uint8_t *A, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                        const uint8_t *B, int64_t ldb, const float *sB, int64_t sb_nb, int64_t sb_kb,
                        int64_t K, const int64_t *ms, const int64_t *ns, int64_t count,
                        double *acc, uint16_t *d, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double v = element(A + m * lda, sA + m * sa_m, sa_kb,
                           B + n * ldb, sB + (n / BLK) * sb_nb, sb_kb, K);
        if (acc)
            acc[i] = v;
        d[i] = dgo_bf16_rne(v);
    }
}

/* Contiguous grouped layout. Row r is produced against expert ids[r] when
 * 0 <= ids[r] < G; rows with any other id are left untouched in D. */
void dgo_grouped_contiguous(const uint8_t *A, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                            const uint8_t *B, int64_t ldb, int64_t b_stride_g,
                            const float *sB, int64_t sb_g, int64_t sb_nb, int64_t sb_kb,
                            const int32_t *ids, uint16_t *D, int64_t ldd,
                            int64_t M_total, int64_t N, int64_t K, int64_t G, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < M_total; ++r)
        for (int64_t n = 0; n < N; ++n) {
            int64_t e = ids[r];
            if (e < 0 || e >= G)
                continue;
            double v = element(A + r * lda, sA + r * sa_m, sa_kb,
                               B + e * b_stride_g + n * ldb, sB + e * sb_g + (n / BLK) * sb_nb,
                               sb_kb, K);
            D[r * ldd + n] = dgo_bf16_rne(v);
        }
}

/* Contiguous grouped layout at points. produced[i] = 0 for a row that is not
 * produced (then acc[i] = NaN and d[i] = 0). */
void dgo_grouped_contiguous_points(const uint8_t *A, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                                   const uint8_t *B, int64_t ldb, int64_t b_stride_g,
                                   const float *sB, int64_t sb_g, int64_t sb_nb, int64_t sb_kb,
                                   const int32_t *ids, int64_t K, int64_t G,
                                   const int64_t *rows, const int64_t *ns, int64_t count,
                                   double *acc, uint16_t *d, uint8_t *produced, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = rows[i], n = ns[i];
        int64_t e = ids[r];
        if (e < 0 || e >= G) {
            produced[i] = 0;
            if (acc)
                acc[i] = NAN;
            d[i] = 0;
            continue;
        }
        double v = element(A + r * lda, sA + r * sa_m, sa_kb,
                           B + e * b_stride_g + n * ldb, sB + e * sb_g + (n / BLK) * sb_nb, sb_kb, K);
        produced[i] = 1;
        if (acc)
            acc[i] = v;
        d[i] = dgo_bf16_rne(v);
    }
}

static int64_t valid_rows(const int32_t *masked_m, int64_t g, int64_t M_max)
{
    int64_t c = masked_m[g];
    if (c < 0)
        c = 0;
    if (c > M_max)
        c = M_max;
    return c;
}

/* Masked grouped layout: group g produces D_g[m, :] for m < clamp(masked_m[g], 0, M_max).
 * A_g = A + g*a_stride_g, sA_g[m,kb] = sA[g*sa_g + m*sa_m + kb*sa_kb], likewise B, sB, D. */
void dgo_grouped_masked(const uint8_t *A, int64_t lda, int64_t a_stride_g,
                        const float *sA, int64_t sa_g, int64_t sa_m, int64_t sa_kb,
                        const uint8_t *B, int64_t ldb, int64_t b_stride_g,
                        const float *sB, int64_t sb_g, int64_t sb_nb, int64_t sb_kb,
                        const int32_t *masked_m, uint16_t *D, int64_t ldd, int64_t d_stride_g,
                        int64_t G, int64_t M_max, int64_t N, int64_t K, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for collapse(3) schedule(static)
    for (int64_t g = 0; g < G; ++g)
        for (int64_t m = 0; m < M_max; ++m)
            for (int64_t n = 0; n < N; ++n) {
                if (m >= valid_rows(masked_m, g, M_max))
                    continue;
                double v = element(A + g * a_stride_g + m * lda, sA + g * sa_g + m * sa_m, sa_kb,
                                   B + g * b_stride_g + n * ldb,
                                   sB + g * sb_g + (n / BLK) * sb_nb, sb_kb, K);
                D[g * d_stride_g + m * ldd + n] = dgo_bf16_rne(v);
            }
}

/* Masked grouped layout at points (gs[i], ms[i], ns[i]); produced[i] = 0 for a
 * row past the group's count. */
void dgo_grouped_masked_points(const uint8_t *A, int64_t lda, int64_t a_stride_g,
                               const float *sA, int64_t sa_g, int64_t sa_m, int64_t sa_kb,
                               const uint8_t *B, int64_t ldb, int64_t b_stride_g,
                               const float *sB, int64_t sb_g, int64_t sb_nb, int64_t sb_kb,
                               const int32_t *masked_m, int64_t M_max, int64_t K,
                               const int64_t *gs, const int64_t *ms, const int64_t *ns, int64_t count,
                               double *acc, uint16_t *d, uint8_t *produced, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t g = gs[i], m = ms[i], n = ns[i];
        if (m >= valid_rows(masked_m, g, M_max)) {
            produced[i] = 0;
            if (acc)
                acc[i] = NAN;
            d[i] = 0;
            continue;
        }
        double v = element(A + g * a_stride_g + m * lda, sA + g * sa_g + m * sa_m, sa_kb,
                           B + g * b_stride_g + n * ldb, sB + g * sb_g + (n / BLK) * sb_nb, sb_kb, K);
        produced[i] = 1;
        if (acc)
            acc[i] = v;
        d[i] = dgo_bf16_rne(v);
    }
}

/* ------------------------------------------------------------------------
 * 1x128 activation quantiser: the step that produces the GEMM's LHS codes
 * and scales from fp32 (or bf16) activations.
 *
 * Per row m and 128-wide K block kb (one LHS scale per 1x128 tile: hotdry.top,
 * "fine-grained scaling core design"):
 *   amax = max |x[m, k]| over the block;
 *   s    = amax / 448 as an fp32 division (the initial scale max_val / 448 of
 *          the rkmt.cn walkthrough, §5.2), or s = 1 when amax == 0;
 *   q    = e4m3 code nearest to clamp(x / s, -448, 448), x / s an fp32
 *          division, ties to the even code (round to nearest rather than
 *          toward zero: lpnh.cn article, §6.3).
 * The sign of a value that rounds to zero is kept (code 0x80 for negatives).
 * Inputs are finite.
 * ------------------------------------------------------------------------ */

/* Nearest e4m3 code to v (|v| <= 448 after the clamp), found by comparing v
 * with every finite non-negative code 0x00..0x7E; on a tie the code with an
 * even mantissa (even code) wins. */
uint8_t dgo_e4m3_encode(float v)
{
    init_table();
    double a = fabs((double)v);
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double best_err = a;                    /* distance to code 0x00 (zero) */
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(dec_table[c] - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(signbit(v) ? (0x80 | best) : best);
}

static float load_x(const void *X, int is_bf16, int64_t i)
{
    if (is_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t *)X)[i] << 16;   /* bf16 is the top half of fp32 */
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    return ((const float *)X)[i];
}

/* X [M, K] (fp32, or bf16 bits when is_bf16), row stride ldx elements.
 * Q [M, K] codes, row stride ldq. S[m, kb] at S[m*s_m + kb*s_kb]. */
void dgo_quantize_1x128(const void *X, int is_bf16, int64_t ldx, int64_t M, int64_t K,
                        uint8_t *Q, int64_t ldq, float *S, int64_t s_m, int64_t s_kb, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t kb = 0; kb < K / BLK; ++kb) {
            float amax = 0.0f;
            for (int64_t k = kb * BLK; k < (kb + 1) * BLK; ++k) {
                float a = fabsf(load_x(X, is_bf16, m * ldx + k));
                if (a > amax)
                    amax = a;
            }
            float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            for (int64_t k = kb * BLK; k < (kb + 1) * BLK; ++k) {
                float v = load_x(X, is_bf16, m * ldx + k) / s;
                Q[m * ldq + k] = dgo_e4m3_encode(v);
            }
            S[m * s_m + kb * s_kb] = s;
        }
}

/* ------------------------------------------------------------------------
 * MoE routing into the contiguous layout, and the way back.
 *
 * Tokens are grouped by expert and laid out one expert after another
 * (regrouping tokens by expert: lpnh.cn article, §5.3), each expert's rows
 * padded to a multiple of 128 so that every aligned 128-row block belongs to
 * one expert (padding to aligned shapes: bhfrc.com article, §4.2), with the
 * group id of every row and the token offsets passed on to the GEMM
 * (rkmt.cn walkthrough, §5.3).
 *
 * Readings: experts in ascending id order, tokens in ascending index order
 * inside an expert; padding rows carry id -1 and token -1; a token whose
 * expert is outside [0, G) is dropped (row -1); rows from the end of the
 * last segment up to M_cap are padding.
 * ------------------------------------------------------------------------ */

/* layout[e] = first row of expert e, layout[G] = rows used (M_total).
 * Returns 0, or -1 when M_cap is too small for the routing. */
int dgo_moe_route_contiguous(const int32_t *expert_of_token, int64_t T, int64_t G,
                             int32_t *row_of_token, int32_t *expert_ids, int32_t *token_of_row,
                             int32_t *layout, int64_t M_cap)
{
    int64_t *count = (int64_t *)calloc((size_t)(G > 0 ? G : 1), sizeof(int64_t));
    int64_t *next = (int64_t *)calloc((size_t)(G > 0 ? G : 1), sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t) {
        int64_t e = expert_of_token[t];
        if (e >= 0 && e < G)
            count[e] += 1;
    }
    int64_t row = 0;
    for (int64_t e = 0; e < G; ++e) {
        layout[e] = (int32_t)row;
        next[e] = row;
        row += (count[e] + BLK - 1) / BLK * BLK;
    }
    layout[G] = (int32_t)row;
    if (row > M_cap) {
        free(count);
        free(next);
        return -1;
    }
    for (int64_t r = 0; r < M_cap; ++r) {
        expert_ids[r] = -1;
        token_of_row[r] = -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        int64_t e = expert_of_token[t];
        if (e < 0 || e >= G) {
            row_of_token[t] = -1;
            continue;
        }
        int64_t r = next[e]++;
        row_of_token[t] = (int32_t)r;
        expert_ids[r] = (int32_t)e;
        token_of_row[r] = (int32_t)t;
    }
    free(count);
    free(next);
    return 0;
}

/* out[t, :] = D[row_of_token[t], :] (bf16 bits); a row index outside
 * [0, d_rows) gives a row of zeros. */
void dgo_moe_unpermute(const uint16_t *D, int64_t ldd, int64_t d_rows, const int32_t *row_of_token,
                       int64_t T, int64_t N, uint16_t *out, int64_t ldo)
{
    for (int64_t t = 0; t < T; ++t) {
        int64_t r = row_of_token[t];
        for (int64_t n = 0; n < N; ++n)
            out[t * ldo + n] = (r >= 0 && r < d_rows) ? D[r * ldd + n] : 0;
    }
}

/* ------------------------------------------------------------------------
 * e5m2 operands. Each operand of the GEMM may instead hold e5m2 codes: 1
 * sign, 5 exponent bits (bias 15), 2 mantissa bits, largest finite 57344,
 * S.11111.00 infinity and S.11111.xx NaN (the two fp8 formats: rkmt.cn
 * walkthrough §2.1; A in e4m3 with B in e5m2 trades precision for range:
 * lpnh.cn article §2.1). The operation is unchanged; a block's scale of an
 * e5m2 operand is amax / 57344.
 *
 * Precision. An e5m2 value is an integer multiple of 2^-16 below 2^16, so a
 * product with e5m2 in it can need up to 64 bits and a 128-term block sum no
 * longer fits binary64. The block sum is therefore taken exactly in 128-bit
 * integers (value * 2^9 for e4m3, value * 2^16 for e5m2) and converted to
 * binary64 once.
 * ------------------------------------------------------------------------ */

double dgo_e5m2_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 2) & 31;
    int f = code & 3;
    double mag;
    if (e == 31)
        return f ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0)
        mag = ldexp((double)f, -16);            /* subnormal: f/4 * 2^-14 */
    else
        mag = ldexp((double)(4 + f), e - 17);   /* (1 + f/4) * 2^(e-15) */
    return s ? -mag : mag;
}

/* fmt 0: e4m3, fmt 1: e5m2. Integer value of a code times 2^(9 or 16). */
static int64_t code_int(uint8_t code, int fmt)
{
    double v = fmt ? dgo_e5m2_decode(code) : dgo_e4m3_decode(code);
    return (int64_t)ldexp(v, fmt ? 16 : 9);     /* exact: the value is a multiple of 2^-16 or 2^-9 */
}

static int code_shift(int fmt) { return fmt ? 16 : 9; }

/* Block partial for formats (fa, fb): exact 128-bit integer sum, one rounding to binary64. */
double dgo_block_partial_fmt(const uint8_t *a, int fa, const uint8_t *b, int fb)
{
    __int128 acc = 0;
    for (int k = 0; k < BLK; ++k)
        acc += (__int128)code_int(a[k], fa) * (__int128)code_int(b[k], fb);
    return ldexp((double)acc, -(code_shift(fa) + code_shift(fb)));
}

static double element_fmt(const uint8_t *a, int fa, const float *sa, int64_t sa_kb,
                          const uint8_t *b, int fb, const float *sb, int64_t sb_kb, int64_t K)
{
    double acc = 0.0;
    for (int64_t kb = 0; kb < K / BLK; ++kb) {
        double partial = dgo_block_partial_fmt(a + kb * BLK, fa, b + kb * BLK, fb);
        double scale = (double)sa[kb * sa_kb] * (double)sb[kb * sb_kb];
        acc += partial * scale;
    }
    return acc;
}

/* Dense NT with operand formats fa (A) and fb (B); otherwise as dgo_gemm_nt. */
void dgo_gemm_nt_fmt(const uint8_t *A, int fa, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                     const uint8_t *B, int fb, int64_t ldb, const float *sB, int64_t sb_nb, int64_t sb_kb,
                     int64_t M, int64_t N, int64_t K, double *acc, uint16_t *D, int64_t ldd, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = element_fmt(A + m * lda, fa, sA + m * sa_m, sa_kb,
                                   B + n * ldb, fb, sB + (n / BLK) * sb_nb, sb_kb, K);
            if (acc)
                acc[m * N + n] = v;
            D[m * ldd + n] = dgo_bf16_rne(v);
        }
}

/* Dense NT with operand formats at chosen output points (ms[i], ns[i]). */
void dgo_gemm_nt_fmt_points(const uint8_t *A, int fa, int64_t lda, const float *sA, int64_t sa_m, int64_t sa_kb,
                            const uint8_t *B, int fb, int64_t ldb, const float *sB, int64_t sb_nb, int64_t sb_kb,
                            int64_t K, const int64_t *ms, const int64_t *ns, int64_t count,
                            double *acc, uint16_t *d, int threads)
{
    init_table();
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double v = element_fmt(A + ms[i] * lda, fa, sA + ms[i] * sa_m, sa_kb,
                               B + ns[i] * ldb, fb, sB + (ns[i] / BLK) * sb_nb, sb_kb, K);
        if (acc)
            acc[i] = v;
        d[i] = dgo_bf16_rne(v);
    }
}
