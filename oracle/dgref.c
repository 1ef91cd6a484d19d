/*
 * dgref.c -- CPU oracle for the FP8 block-scaled NT GEMM (dense, contiguous-grouped,
 * masked-grouped).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * What it computes (the method's own definition, written out plainly):
 *
 *   C[m,n] = bf16_rne( sum_kb  sA[m,kb] * sB_g[n/128, kb] *
 *                      sum_{k in block kb}  dec(A[m,k]) * dec(B_g[n,k]) )
 *
 *   - NT layout: A is M x K row-major, B is stored N x K row-major (the RHS is
 *     transposed); DeepGEMM page on turtlesai.it, technical summary paragraph.
 *   - fine-grained scaling: one fp32 scale per 1x128 block of A and per 128x128 block
 *     of B; same paragraph ("ridimensionamento a grana fine") and the chattools.cn
 *     article, section on core design ideas.
 *   - two-level accumulation: each 128-deep K block is summed on its own, scaled, and
 *     then added into a separate higher-precision accumulator (same two sources).
 *   - BF16 output: aisharenet.com/ja usage guide, section "basic FP8 GEMM".
 *   - grouping on M only, experts share N and K: aisharenet.com/ja usage guide,
 *     section on grouped GEMM for MoE; contiguous and masked layouts: flashmla.org/zh
 *     page, section "DeepGEMM performance", and the usage guide's sections 2 and 3.
 *
 * Operand formats: E4M3 ("fn") by default; either operand may instead be E5M2, the
 * other 8-bit format the aisharenet.com/ja usage guide names for the inputs (main
 * functions, section 1).
 *
 * Precision: the block partial is exact.  With two E4M3 operands it is summed in fp64,
 * which is exact (each product has at most 8 significant bits and magnitude in
 * [2^-18, 448^2]; 128 of them stay below 2^25, i.e. within 43 bits).  An E5M2 operand
 * widens the range (down to 2^-16, up to 57344), so such blocks are summed exactly in
 * 128-bit integers (every E4M3 value is an integer times 2^-9, every E5M2 value an
 * integer times 2^-16) and rounded once to fp64.  sA*sB is exact in fp64 (24+24 bits).
 * The scaled term is rounded once to fp64, the K-block sum runs in fp64 in kb order
 * 0,1,2,..., and the result is rounded once, directly from fp64, to bf16 with
 * round-to-nearest-even.
 *
 * Readings where the pages are silent (each one is listed with its reason in the
 * design notes of this repository):
 *   - K need not be a multiple of 128 here: the last block is short and uses scale
 *     column floor(k/128).
 *   - N need not be a multiple of 128: sB has ceil(N/128) rows; column n uses row n/128.
 *   - contiguous routing: row m is written iff 0 <= group_idx[m] < G and
 *     group_idx[m] == group_idx[128*floor(m/128)]; other rows are left untouched.
 *   - masked routing: group g writes rows [0, clamp(masked_m[g], 0, cap)); all other
 *     rows of C are left untouched, and A rows past that count are never read.
 *
 * Parity pins live in tests/ (worked example, exact-rational brute force, integer
 * inputs, power-of-two scaling, group-order independence, untouched masked rows,
 * reductions between the three forms, NumPy fp64 matmul with unit scales; for the
 * quantiser, torch's fp8 rounding and the scale's definition).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DGREF_BLOCK 128

/* OCP 8-bit floating point, E4M3 ("fn": finite, no infinities).  Sign bit, 4-bit
 * exponent with bias 7, 3-bit mantissa.  Exponent field 0 is subnormal: m * 2^-9.
 * S.1111.111 is NaN; every other code is finite; the largest is 0x7E = 448. */
double dgref_e4m3fn_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* 0.m * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10);       /* 1.m * 2^(e-7) */
    return sign ? -v : v;
}

/* OCP 8-bit floating point, E5M2.  Sign bit, 5-bit exponent with bias 15, 2-bit
 * mantissa.  Exponent field 0 is subnormal: m * 2^-16.  Exponent field 31 holds the
 * infinities (mantissa 0) and NaNs (mantissa != 0); the largest finite is 0x7B = 57344. */
double dgref_e5m2_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 2) & 0x1F;
    int m = code & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);                /* 0.m * 2^(1-15) */
    else
        v = ldexp((double)(4 + m), e - 17);       /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 (8 significant bits, 8 exponent bits, bias 127),
 * ties to even, in one step from the double value.  NaN -> 0x7FC0.  Overflow past the
 * largest finite bf16 rounds to infinity, as round-to-nearest requires. */
uint16_t dgref_bf16_rne(double x)
{
    union { float f; uint32_t u; } cv;
    double ax, q, r, fl, y;
    int e;
    if (isnan(x))
        return 0x7FC0;
    ax = fabs(x);
    if (ax == 0.0) {
        cv.f = (float)x;                          /* keeps the sign of zero */
        return (uint16_t)(cv.u >> 16);
    }
    frexp(ax, &e);                                /* ax = f * 2^e, f in [0.5, 1) */
    if (e < -125)
        e = -125;                                 /* subnormal bf16: fixed quantum 2^-133 */
    q = ldexp(1.0, e - 8);                        /* spacing of bf16 values near ax */
    r = ax / q;                                   /* exact: division by a power of two */
    fl = floor(r);
    if (r - fl > 0.5 || (r - fl == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    y = fl * q;
    if (y >= ldexp(1.0, 128))
        return (uint16_t)(x < 0 ? 0xFF80 : 0x7F80);
    cv.f = (float)(x < 0 ? -y : y);               /* exact: y has at most 8 significant bits */
    return (uint16_t)(cv.u >> 16);
}

#define DGREF_E4M3 0
#define DGREF_E5M2 1

/* Decoded values per format, and for the integer path each finite value as an integer
 * times 2^-LSB_EXP (E4M3: 2^-9, E5M2: 2^-16); the integer table is only read for finite
 * codes (non-finite codes send the element down the fp64 path). */
static double g_dec[2][256];
static int64_t g_int[2][256];
static int g_fin[2][256];
static const int g_lsb_exp[2] = {9, 16};
static int g_dec_ready = 0;

static void build_decode_table(void)
{
    int c, f;
    if (g_dec_ready)
        return;
    for (c = 0; c < 256; ++c) {
        g_dec[DGREF_E4M3][c] = dgref_e4m3fn_decode((uint8_t)c);
        g_dec[DGREF_E5M2][c] = dgref_e5m2_decode((uint8_t)c);
    }
    for (f = 0; f < 2; ++f)
        for (c = 0; c < 256; ++c) {
            double v = g_dec[f][c];
            g_fin[f][c] = isfinite(v);
            g_int[f][c] = g_fin[f][c] ? (int64_t)ldexp(v, g_lsb_exp[f]) : 0;  /* exact */
        }
    g_dec_ready = 1;
}

/* The exact partial of one K block when an operand is E5M2: the integer sum of the
 * integer products, then one rounding to fp64.  Falls back to the fp64 sum (which then
 * carries the infinities/NaNs) when a code is not finite. */
static double block_partial_wide(const uint8_t *a, int fa, const uint8_t *b, int fb,
                                 int64_t k0, int64_t k1)
{
    __int128 s = 0;
    int64_t k;
    double partial = 0.0;
    for (k = k0; k < k1; ++k)
        if (!g_fin[fa][a[k]] || !g_fin[fb][b[k]]) {
            for (k = k0; k < k1; ++k)
                partial += g_dec[fa][a[k]] * g_dec[fb][b[k]];
            return partial;
        }
    for (k = k0; k < k1; ++k)
        s += (__int128)g_int[fa][a[k]] * (__int128)g_int[fb][b[k]];   /* < 2^64 each */
    /* |s| < 2^71: split into two exactly representable halves, rounded once on adding */
    {
        int64_t hi = (int64_t)(s >> 32);
        uint64_t lo = (uint64_t)(s & 0xFFFFFFFFu);
        double v = ldexp((double)hi, 32) + (double)lo;   /* one rounding */
        return ldexp(v, -(g_lsb_exp[fa] + g_lsb_exp[fb]));
    }
}

/* The unrounded fp64 result of one output element: the two-level sum above. */
static double element_f64(const uint8_t *a_row, int fa, const float *sa_row,
                          const uint8_t *b_row, int fb, const float *sb_row, int64_t K)
{
    int64_t nkb = (K + DGREF_BLOCK - 1) / DGREF_BLOCK;
    double acc = 0.0;
    int64_t kb, k;
    for (kb = 0; kb < nkb; ++kb) {
        int64_t k0 = kb * DGREF_BLOCK;
        int64_t k1 = k0 + DGREF_BLOCK < K ? k0 + DGREF_BLOCK : K;
        double partial = 0.0;
        double s;
        if (fa == DGREF_E4M3 && fb == DGREF_E4M3) {
            for (k = k0; k < k1; ++k)
                partial += g_dec[fa][a_row[k]] * g_dec[fb][b_row[k]];
        } else {
            partial = block_partial_wide(a_row, fa, b_row, fb, k0, k1);
        }
        s = (double)sa_row[kb] * (double)sb_row[kb];
        acc += partial * s;
    }
    return acc;
}

/* One output row against one group's B.  acc_out (optional) receives the unrounded
 * fp64 values, c_out (optional) the bf16 bits. */
static void one_row(const uint8_t *a_row, int fa, const float *sa_row, const uint8_t *B,
                    int fb, const float *sB, int64_t N, int64_t K, uint16_t *c_out,
                    double *acc_out)
{
    int64_t nkb = (K + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t n;
    for (n = 0; n < N; ++n) {
        const uint8_t *b_row = B + n * K;
        const float *sb_row = sB + (n / DGREF_BLOCK) * nkb;
        double v = element_f64(a_row, fa, sa_row, b_row, fb, sb_row, K);
        if (acc_out)
            acc_out[n] = v;
        if (c_out)
            c_out[n] = dgref_bf16_rne(v);
    }
}

static int valid_formats(int fa, int fb)
{
    return (fa == DGREF_E4M3 || fa == DGREF_E5M2) && (fb == DGREF_E4M3 || fb == DGREF_E5M2);
}

int dgref_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Dense: C (M x N bf16) = A (M x K) x B (N x K)^T with the block scales; fa / fb are
 * the operand formats (0: E4M3, 1: E5M2).  acc (optional, M x N doubles) receives the
 * unrounded values.  Returns -1 for an unknown format, else 0. */
int dgref_gemm_fp8_nt_fmt(const uint8_t *A, int fa, const float *sA, const uint8_t *B,
                          int fb, const float *sB, uint16_t *C, double *acc,
                          int64_t M, int64_t N, int64_t K)
{
    int64_t nkb = (K + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t m;
    if (!valid_formats(fa, fb))
        return -1;
    build_decode_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m)
        one_row(A + m * K, fa, sA + m * nkb, B, fb, sB, N, K,
                C ? C + m * N : 0, acc ? acc + m * N : 0);
    return 0;
}

void dgref_gemm_fp8_nt(const uint8_t *A, const float *sA, const uint8_t *B,
                       const float *sB, uint16_t *C, double *acc,
                       int64_t M, int64_t N, int64_t K)
{
    dgref_gemm_fp8_nt_fmt(A, DGREF_E4M3, sA, B, DGREF_E4M3, sB, C, acc, M, N, K);
}

/* Contiguous grouped: rows of all groups concatenated (M_total x K); B is G x N x K,
 * sB is G x ceil(N/128) x ceil(K/128); group_idx is one int32 per row. */
int dgref_grouped_contiguous_fmt(const uint8_t *A, int fa, const float *sA,
                                 const uint8_t *B, int fb, const float *sB,
                                 const int32_t *group_idx, uint16_t *C, double *acc,
                                 int64_t M_total, int64_t N, int64_t K, int64_t G)
{
    int64_t nkb = (K + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t nnb = (N + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t m;
    if (!valid_formats(fa, fb))
        return -1;
    build_decode_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M_total; ++m) {
        int32_t g = group_idx[m];
        int32_t lead = group_idx[(m / DGREF_BLOCK) * DGREF_BLOCK];
        if (g < 0 || g >= G || g != lead)
            continue;                             /* row left untouched */
        one_row(A + m * K, fa, sA + m * nkb, B + (int64_t)g * N * K, fb,
                sB + (int64_t)g * nnb * nkb, N, K, C ? C + m * N : 0, acc ? acc + m * N : 0);
    }
    return 0;
}

void dgref_grouped_contiguous(const uint8_t *A, const float *sA, const uint8_t *B,
                              const float *sB, const int32_t *group_idx, uint16_t *C,
                              double *acc, int64_t M_total, int64_t N, int64_t K,
                              int64_t G)
{
    dgref_grouped_contiguous_fmt(A, DGREF_E4M3, sA, B, DGREF_E4M3, sB, group_idx, C, acc,
                                 M_total, N, K, G);
}

/* Masked grouped: A is G x cap x K, C is G x cap x N; group g computes its first
 * clamp(masked_m[g], 0, cap) rows and leaves the rest of C untouched. */
int dgref_grouped_masked_fmt(const uint8_t *A, int fa, const float *sA, const uint8_t *B,
                             int fb, const float *sB, const int32_t *masked_m, uint16_t *C,
                             double *acc, int64_t G, int64_t cap, int64_t N, int64_t K)
{
    int64_t nkb = (K + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t nnb = (N + DGREF_BLOCK - 1) / DGREF_BLOCK;
    int64_t i;
    if (!valid_formats(fa, fb))
        return -1;
    build_decode_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < G * cap; ++i) {
        int64_t g = i / cap, m = i % cap;
        int64_t valid = masked_m[g];
        if (valid < 0)
            valid = 0;
        if (valid > cap)
            valid = cap;
        if (m >= valid)
            continue;                             /* row left untouched */
        one_row(A + i * K, fa, sA + i * nkb, B + g * N * K, fb, sB + g * nnb * nkb, N, K,
                C ? C + i * N : 0, acc ? acc + i * N : 0);
    }
    return 0;
}

void dgref_grouped_masked(const uint8_t *A, const float *sA, const uint8_t *B,
                          const float *sB, const int32_t *masked_m, uint16_t *C,
                          double *acc, int64_t G, int64_t cap, int64_t N, int64_t K)
{
    dgref_grouped_masked_fmt(A, DGREF_E4M3, sA, B, DGREF_E4M3, sB, masked_m, C, acc, G, cap,
                             N, K);
}

/* ------------------------------------------------------------------------------------
 * Quantisation to fp8 with block scales -- the casting step the turtlesai.it summary
 * (technical paragraph) leaves to the user, in the two block shapes of the method's
 * fine-grained scaling: one scale per 1x128 block (activations, per row and K block)
 * and one per 128x128 block (weights).  Per block: amax = max |x| in fp32; scale =
 * amax / FMAX in fp32 (FMAX = 448 for E4M3, 57344 for E5M2; 1 when amax is 0); each
 * code is the nearest fp8 value to x / scale (an fp32 division), ties to the even code,
 * after saturating to +-FMAX.  Inputs are finite.  K is a multiple of 128; the row
 * count of the 128x128 form need not be (the last block row holds the rows that exist).
 */

/* The finite fp8 code nearest to v (saturated to the largest finite value), ties to
 * the code with an even mantissa: a search over every positive finite code. */
static uint8_t encode_fp8_nearest(double v, int fmt)
{
    double maxv = fmt == DGREF_E5M2 ? 57344.0 : 448.0;
    double a = fabs(v), best_d = INFINITY;
    int c, best = 0;
    if (a > maxv)
        a = maxv;
    for (c = 0; c < 128; ++c) {
        double d = g_dec[fmt][c], diff;
        if (!isfinite(d))
            continue;
        diff = fabs(a - d);
        if (diff < best_d || (diff == best_d && (c & 1) == 0)) {
            best_d = diff;
            best = c;
        }
    }
    if (signbit(v))
        best |= 0x80;
    return (uint8_t)best;
}

static float block_scale(float amax, int fmt)
{
    float fmax = fmt == DGREF_E5M2 ? 57344.0f : 448.0f;
    return amax == 0.0f ? 1.0f : amax / fmax;
}

/* x / scale as an IEEE fp32 division.  A non-zero amax gives a zero scale only when
 * amax / FMAX underflows (fp32 blocks with amax at most FMAX * 2^-150); then x / 0 is
 * +-infinity, which the encoder saturates, and 0 / 0 is read as a zero with the sign of
 * x (the sign of a zero quotient follows x everywhere else too). */
static float block_quotient(float x, float scale)
{
    float q = x / scale;
    return isnan(q) ? copysignf(0.0f, x) : q;
}

/* X rows x K fp32 -> Q rows x K codes, S rows x K/128 scales.  Returns -1 for an
 * unknown format or K not a multiple of 128, else 0. */
int dgref_quantize_1x128(const float *X, int64_t rows, int64_t K, int fmt, uint8_t *Q,
                         float *S)
{
    int64_t nkb = K / DGREF_BLOCK, r;
    if ((fmt != DGREF_E4M3 && fmt != DGREF_E5M2) || K % DGREF_BLOCK != 0)
        return -1;
    build_decode_table();
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t kb, k;
        for (kb = 0; kb < nkb; ++kb) {
            const float *x = X + r * K + kb * DGREF_BLOCK;
            float amax = 0.0f, scale;
            for (k = 0; k < DGREF_BLOCK; ++k)
                if (fabsf(x[k]) > amax)
                    amax = fabsf(x[k]);
            scale = block_scale(amax, fmt);
            S[r * nkb + kb] = scale;
            for (k = 0; k < DGREF_BLOCK; ++k) {
                float q = block_quotient(x[k], scale);
                Q[r * K + kb * DGREF_BLOCK + k] = encode_fp8_nearest((double)q, fmt);
            }
        }
    }
    return 0;
}

/* X rows x K fp32 -> Q rows x K codes, S ceil(rows/128) x K/128 scales. */
int dgref_quantize_128x128(const float *X, int64_t rows, int64_t K, int fmt, uint8_t *Q,
                           float *S)
{
    int64_t nkb = K / DGREF_BLOCK, nrb = (rows + DGREF_BLOCK - 1) / DGREF_BLOCK, b;
    if ((fmt != DGREF_E4M3 && fmt != DGREF_E5M2) || K % DGREF_BLOCK != 0)
        return -1;
    build_decode_table();
#pragma omp parallel for schedule(static)
    for (b = 0; b < nrb * nkb; ++b) {
        int64_t rb = b / nkb, kb = b % nkb, r, k;
        int64_t r0 = rb * DGREF_BLOCK, r1 = r0 + DGREF_BLOCK < rows ? r0 + DGREF_BLOCK : rows;
        int64_t k0 = kb * DGREF_BLOCK;
        float amax = 0.0f, scale;
        for (r = r0; r < r1; ++r)
            for (k = k0; k < k0 + DGREF_BLOCK; ++k)
                if (fabsf(X[r * K + k]) > amax)
                    amax = fabsf(X[r * K + k]);
        scale = block_scale(amax, fmt);
        S[rb * nkb + kb] = scale;
        for (r = r0; r < r1; ++r)
            for (k = k0; k < k0 + DGREF_BLOCK; ++k) {
                float q = block_quotient(X[r * K + k], scale);
                Q[r * K + k] = encode_fp8_nearest((double)q, fmt);
            }
    }
    return 0;
}

/* Element-wise helpers for the tests. */
void dgref_bf16_rne_array(const double *x, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = dgref_bf16_rne(x[i]);
}

void dgref_e4m3fn_decode_array(const uint8_t *codes, double *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = dgref_e4m3fn_decode(codes[i]);
}

void dgref_e5m2_decode_array(const uint8_t *codes, double *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = dgref_e5m2_decode(codes[i]);
}

/* fp8 encoding (nearest, ties to even, saturating) of each value, for the tests. */
void dgref_encode_fp8_array(const double *x, uint8_t *out, int64_t n, int fmt)
{
    int64_t i;
    build_decode_table();
    for (i = 0; i < n; ++i)
        out[i] = encode_fp8_nearest(x[i], fmt);
}
