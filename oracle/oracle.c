/*
 * Blockwise-scaled FP8 oracle: a plain, slow, deliberately obvious CPU implementation of what the
 * blockwise FP8 linear-layer path computes.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the benchmark's CPU
 * baseline leg may load or call this library. It shares no code with the HIP path.
 *
 * Sources (pytorch/ao pull-request pages on blockwise FP8 training):
 *   [ROCm]  "Enable blockwise FP8 dense training kernels on ROCm":
 *           - description: FP8_MAX is the float8 format's finfo max (448 for float8_e4m3fn);
 *           - quantization-correctness table: act_quant_lhs / act_quant_rhs / weight_quant_rhs with
 *             block_size 128;
 *           - root-cause comment: the LHS activation quantizer stores *reciprocal* scales into a
 *             column-major [M, K/128] tensor, so a row index >= M would alias into the next
 *             K-block column.
 *   [Mask]  "Mask a_s/b_s scale loads in blockwise FP8 training GEMM kernels", Summary and Fix:
 *           the 1x128_128x128 and 1x128_128x1 GEMMs read one a_s value per (row, K-block) and one
 *           b_s value per (K-block, N-block) or (K-block, column); rows >= M and columns >= N take
 *           no part.
 *   [OFP8]  The OCP 8-bit floating point specification, E4M3 encoding (bias 7, no infinities,
 *           S.1111.111 is NaN, max normal 448, min subnormal 2^-9).
 *   [FNUZ]  The float8_e4m3fnuz format the ROCm page names for MI300X (its description and test
 *           log: FP8 max 240): 1 sign, 4 exponent bits with bias 8, 3 mantissa bits, no
 *           infinities and no negative zero -- the bit pattern 1.0000.000 (0x80) is the only NaN,
 *           0x7F is the largest finite value 240, the smallest normal is 2^-7 and the smallest
 *           subnormal 2^-10.
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - eps clamp on the group amax: 1e-12f, applied before both divisions;
 *   - stored scale s = fl32(amax_c / FP8_MAX), the dequantization multiplier ("reciprocal scale");
 *   - codes q = enc(clamp(fl32(x * fl32(FP8_MAX / amax_c)), -FP8_MAX, FP8_MAX)): multiply by the
 *     quantization multiplier, then round to nearest even and saturate;
 *   - FP8_MAX is the finfo max of the chosen element format: 448 for e4m3fn (the default), 240
 *     for e4m3fnuz ([ROCm] description: the limits follow torch.finfo(dtype) and both formats are
 *     accepted); every other step is the same for both;
 *   - partial groups at a tensor edge use only their valid elements.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fexcess-precision=standard -fopenmp.
 * On x86-64 every float expression below is one IEEE binary32 operation, correctly rounded.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP_EPS 1e-12f /* reading: amax clamp so an all-zero group has a finite, non-zero scale */
#define BLOCK 128        /* [ROCm] quantization table: block_size = 128 */

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static float bf16_value(uint16_t bits)
{
    /* A bf16 is the high half of a binary32: widening is exact. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---------------------------------------------------------------- element codecs */

/*
 * The two 8-bit formats differ only in their exponent bias, their largest finite code and their
 * treatment of zero and NaN:
 *                 bias  largest finite       NaN codes          zero codes
 *   e4m3fn [OFP8]   7   0x7E = 448           0x7F, 0xFF         0x00 (+0), 0x80 (-0)
 *   e4m3fnuz[FNUZ]  8   0x7F = 240           0x80               0x00 only
 */
struct e4m3_format {
    int bias;
    uint8_t max_code;
    double max_value;
    int negative_zero;      /* 1: a negative value that rounds to zero keeps its sign (0x80) */
};

static const struct e4m3_format FMT_FN = {7, 0x7E, 448.0, 1};
static const struct e4m3_format FMT_FNUZ = {8, 0x7F, 240.0, 0};

static const struct e4m3_format* format_of(int fmt)
{
    return fmt == ORACLE_FMT_E4M3FNUZ ? &FMT_FNUZ : &FMT_FN;
}

static double decode_generic(uint8_t code, const struct e4m3_format* f)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (f->negative_zero) {
        if (e == 0xF && m == 0x7)
            return NAN;                              /* [OFP8] S.1111.111 */
    } else if (code == 0x80) {
        return NAN;                                  /* [FNUZ] the negative-zero pattern */
    }
    if (e == 0)
        mag = ldexp((double)m, 1 - f->bias - 3);     /* subnormal: m/8 * 2^(1 - bias) */
    else
        mag = ldexp(1.0 + m / 8.0, e - f->bias);     /* normal: (1 + m/8) * 2^(e - bias) */
    return sign ? -mag : mag;
}

/*
 * Round-to-nearest-even, saturating encode of a finite binary32 value.
 * With emin = 1 - bias the smallest normal exponent, the representable magnitudes in the binade
 * [2^e, 2^(e+1)) are spaced 2^(e-3) apart for e >= emin; below 2^emin the spacing stays
 * 2^(emin-3) (subnormals). Magnitudes >= the largest finite value saturate to it.
 */
static uint8_t encode_generic(float v, const struct e4m3_format* f)
{
    const int emin = 1 - f->bias;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int e, ex, code;
    double quantum, r, fl, frac;
    int64_t n;

    if (a >= f->max_value)
        return (uint8_t)(sign | f->max_code);

    if (a == 0.0) {
        e = emin;
    } else {
        (void)frexp(a, &ex);    /* a = g * 2^ex, g in [0.5, 1): floor(log2 a) = ex - 1 */
        e = ex - 1;
        if (e < emin)
            e = emin;
    }
    quantum = ldexp(1.0, e - 3);
    r = a / quantum;            /* exact: a has 24 significant bits, quantum is a power of two */
    fl = floor(r);
    frac = r - fl;
    n = (int64_t)fl;
    if (frac > 0.5 || (frac == 0.5 && (n & 1)))
        n += 1;                 /* nearest, ties to even */

    if (n >= 16) {              /* mantissa carried into the next binade */
        n = 8;
        e += 1;
    }
    /* Now n in [8, 15] is a normal significand (1 + (n-8)/8) at exponent e, or e == emin and
     * n in [0, 7] is a subnormal (or zero), whose exponent field is 0. Rounding cannot pass the
     * largest finite value: a is below it and the next step above it needs a half step more. */
    if (n < 8)
        code = (int)n;
    else
        code = ((e + f->bias) << 3) + (int)(n - 8);
    if (code == 0 && !f->negative_zero)
        return 0x00;            /* [FNUZ] zero has no sign */
    return (uint8_t)(sign | code);
}

double oracle_e4m3_decode(uint8_t code) { return decode_generic(code, &FMT_FN); }
uint8_t oracle_e4m3_encode(float v) { return encode_generic(v, &FMT_FN); }
double oracle_e4m3fnuz_decode(uint8_t code) { return decode_generic(code, &FMT_FNUZ); }
uint8_t oracle_e4m3fnuz_encode(float v) { return encode_generic(v, &FMT_FNUZ); }

void oracle_fp8_encode_array(int fmt, const float* v, uint8_t* codes, int64_t n)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        codes[i] = encode_generic(v[i], f);
}

void oracle_fp8_encode_bits(int fmt, uint32_t first, uint8_t* codes, int64_t n)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i;
        float x;
        memcpy(&x, &u, sizeof x);
        codes[i] = isnan(x) ? 0xFF : encode_generic(x, f);
    }
}

void oracle_e4m3_encode_array(const float* v, uint8_t* codes, int64_t n)
{
    oracle_fp8_encode_array(ORACLE_FMT_E4M3FN, v, codes, n);
}

void oracle_e4m3_encode_bits(uint32_t first, uint8_t* codes, int64_t n)
{
    oracle_fp8_encode_bits(ORACLE_FMT_E4M3FN, first, codes, n);
}

/* ---------------------------------------------------------------- one group */

/*
 * The per-group quantization step shared by all three groupings: the group's n valid values are
 * given in vals[]; their codes (in format f) are written to codes[] and the stored
 * (dequantization) scale is returned.
 */
static float quantize_group(const float* vals, int64_t n, uint8_t* codes,
                            const struct e4m3_format* f)
{
    const float FP8_MAX = (float)f->max_value; /* [ROCm] description: finfo(dtype).max */
    float amax = 0.0f, amax_c, s, m;
    int64_t i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(vals[i]);
        if (a > amax)
            amax = a;
    }
    amax_c = amax > GROUP_EPS ? amax : GROUP_EPS;
    s = amax_c / FP8_MAX;   /* stored "reciprocal" scale: x ~= dec(q) * s */
    m = FP8_MAX / amax_c;   /* quantization multiplier */
    for (i = 0; i < n; ++i) {
        float v = vals[i] * m;
        if (v > FP8_MAX)
            v = FP8_MAX;
        if (v < -FP8_MAX)
            v = -FP8_MAX;
        codes[i] = encode_generic(v, f);
    }
    return s;
}

/* ---------------------------------------------------------------- quantizers */

int oracle_quantize_lhs(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* a_s, int fmt)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t Kb, m;
    if (M < 0 || K < 0 || ldx < K || ldq < K)
        return -1;
    if (M == 0 || K == 0)
        return 0;
    if (!x || !q || !a_s)
        return -1;
    Kb = cdiv(K, BLOCK);
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        float vals[BLOCK];
        uint8_t codes[BLOCK];
        int64_t kb, k;
        for (kb = 0; kb < Kb; ++kb) {
            int64_t k0 = kb * BLOCK;
            int64_t n = (K - k0) < BLOCK ? (K - k0) : BLOCK;
            for (k = 0; k < n; ++k)
                vals[k] = bf16_value(x[m * ldx + k0 + k]);
            /* column-major [M, Kb]: element (m, kb) lives at kb * M + m */
            a_s[kb * M + m] = quantize_group(vals, n, codes, f);
            for (k = 0; k < n; ++k)
                q[m * ldq + k0 + k] = codes[k];
        }
    }
    return 0;
}

int oracle_quantize_rhs(const uint16_t* x, int64_t K, int64_t N, int64_t ldx,
                        uint8_t* qT, int64_t ldqT, float* s, int fmt)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t Kb, col;
    if (K < 0 || N < 0 || ldx < N || ldqT < K)
        return -1;
    if (K == 0 || N == 0)
        return 0;
    if (!x || !qT || !s)
        return -1;
    Kb = cdiv(K, BLOCK);
#pragma omp parallel for schedule(static)
    for (col = 0; col < N; ++col) {
        float vals[BLOCK];
        uint8_t codes[BLOCK];
        int64_t kb, k;
        for (kb = 0; kb < Kb; ++kb) {
            int64_t k0 = kb * BLOCK;
            int64_t n = (K - k0) < BLOCK ? (K - k0) : BLOCK;
            for (k = 0; k < n; ++k)
                vals[k] = bf16_value(x[(k0 + k) * ldx + col]);
            s[kb * N + col] = quantize_group(vals, n, codes, f);
            for (k = 0; k < n; ++k)
                qT[col * ldqT + k0 + k] = codes[k];
        }
    }
    return 0;
}

int oracle_quantize_weight_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s,
                                   int fmt)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t Nb, Kb, blk;
    if (N < 0 || K < 0 || ldw < K || ldq < K || (qT && ldqT < N))
        return -1;
    if (N == 0 || K == 0)
        return 0;
    if (!w || !q || !s)
        return -1;
    Nb = cdiv(N, BLOCK);
    Kb = cdiv(K, BLOCK);
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < Nb * Kb; ++blk) {
        int64_t nb = blk / Kb, kb = blk % Kb;
        int64_t n0 = nb * BLOCK, k0 = kb * BLOCK;
        int64_t rn = (N - n0) < BLOCK ? (N - n0) : BLOCK;
        int64_t rk = (K - k0) < BLOCK ? (K - k0) : BLOCK;
        float* vals = (float*)malloc(sizeof(float) * BLOCK * BLOCK);
        uint8_t* codes = (uint8_t*)malloc(BLOCK * BLOCK);
        int64_t i, j;
        for (i = 0; i < rn; ++i)
            for (j = 0; j < rk; ++j)
                vals[i * rk + j] = bf16_value(w[(n0 + i) * ldw + k0 + j]);
        s[nb * Kb + kb] = quantize_group(vals, rn * rk, codes, f);
        for (i = 0; i < rn; ++i)
            for (j = 0; j < rk; ++j) {
                q[(n0 + i) * ldq + k0 + j] = codes[i * rk + j];
                if (qT)
                    qT[(k0 + j) * ldqT + n0 + i] = codes[i * rk + j];
            }
        free(vals);
        free(codes);
    }
    return 0;
}

/* ---------------------------------------------------------------- scaled GEMMs */

/*
 * C[m, n] = sum over K-blocks kb of  a_s[m, kb] * b_scale(kb, n) * sum_{k in kb, k < K} A[m,k] B[n,k]
 * with A, B the decoded fp8 values (both in format fmt). Products of two e4m3 values are exact in
 * fp64 and a K-block's partial sum of at most 128 of them is exact too (their magnitudes span under
 * 2^45); only the outer sum over K-blocks rounds, at fp64.
 * bscale_kind 0: 128x128 blocks via (stride_nb, stride_kb); 1: per column, b_s[kb * N + n].
 */
static int gemm_rows(const uint8_t* a, int64_t lda, const float* a_s,
                     const uint8_t* b, int64_t ldb, const float* b_s,
                     int bscale_kind, int64_t bs_stride_nb, int64_t bs_stride_kb,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t nrows, double* out, int fmt)
{
    const struct e4m3_format* f = format_of(fmt);
    int64_t Kb, r;
    double* bdec;
    double table[256];
    int i;
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || lda < K || ldb < K)
        return -1;
    if (nrows == 0 || N == 0)
        return 0;
    if (!out || !rows)
        return -1;
    for (r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return -2;
    if (K == 0) {
        memset(out, 0, sizeof(double) * nrows * N);
        return 0;
    }
    if (!a || !a_s || !b || !b_s)
        return -1;
    Kb = cdiv(K, BLOCK);
    for (i = 0; i < 256; ++i)
        table[i] = decode_generic((uint8_t)i, f);

    /* decode B once: [N, K] doubles */
    bdec = (double*)malloc(sizeof(double) * N * K);
    if (!bdec)
        return -3;
    {
        int64_t nn;
#pragma omp parallel for schedule(static)
        for (nn = 0; nn < N; ++nn) {
            int64_t k;
            for (k = 0; k < K; ++k)
                bdec[nn * K + k] = table[b[nn * ldb + k]];
        }
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < nrows; ++r) {
        int64_t m = rows[r];
        double* adec = (double*)malloc(sizeof(double) * K);
        int64_t n, k, kb;
        for (k = 0; k < K; ++k)
            adec[k] = table[a[m * lda + k]];
        for (n = 0; n < N; ++n) {
            double total = 0.0;
            const double* brow = bdec + n * K;
            for (kb = 0; kb < Kb; ++kb) {
                int64_t k0 = kb * BLOCK;
                int64_t k1 = (k0 + BLOCK) < K ? (k0 + BLOCK) : K;
                double part = 0.0, sa, sb;
                for (k = k0; k < k1; ++k)
                    part += adec[k] * brow[k];
                sa = (double)a_s[kb * M + m];
                if (bscale_kind == 0)
                    sb = (double)b_s[(n / BLOCK) * bs_stride_nb + kb * bs_stride_kb];
                else
                    sb = (double)b_s[kb * N + n];
                total += sa * sb * part;
            }
            out[r * N + n] = total;
        }
        free(adec);
    }
    free(bdec);
    return 0;
}

int oracle_gemm_1x128_128x128(const uint8_t* a, int64_t lda, const float* a_s,
                              const uint8_t* b, int64_t ldb, const float* b_s,
                              int64_t bs_stride_nb, int64_t bs_stride_kb,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t* rows, int64_t nrows, double* out, int fmt)
{
    return gemm_rows(a, lda, a_s, b, ldb, b_s, 0, bs_stride_nb, bs_stride_kb, M, N, K,
                     rows, nrows, out, fmt);
}

int oracle_gemm_1x128_128x1(const uint8_t* a, int64_t lda, const float* a_s,
                            const uint8_t* b, int64_t ldb, const float* b_s,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t* rows, int64_t nrows, double* out, int fmt)
{
    return gemm_rows(a, lda, a_s, b, ldb, b_s, 1, 0, 0, M, N, K, rows, nrows, out, fmt);
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
