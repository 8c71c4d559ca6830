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
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - eps clamp on the group amax: 1e-12f, applied before both divisions;
 *   - stored scale s = fl32(amax_c / 448), the dequantization multiplier ("reciprocal scale");
 *   - codes q = e4m3(clamp(fl32(x * fl32(448 / amax_c)), -448, 448)): multiply by the quantization
 *     multiplier, then round to nearest even and saturate;
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

#define FP8_MAX 448.0f /* [ROCm] description: finfo(float8_e4m3fn).max */
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

/* ---------------------------------------------------------------- e4m3fn codec [OFP8] */

double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;                          /* S.1111.111 */
    if (e == 0)
        mag = ldexp((double)m, -9);          /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);   /* normal: (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/*
 * Round-to-nearest-even, saturating encode of a finite binary32 value.
 * The representable magnitudes in the binade [2^e, 2^(e+1)) are spaced 2^(e-3) apart for e >= -6;
 * below 2^-6 the spacing stays 2^-9 (subnormals). Magnitudes >= 448 saturate to 448.
 */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int e, ex;
    double quantum, r, fl, frac;
    int64_t n;

    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);

    if (a == 0.0) {
        e = -6;
    } else {
        (void)frexp(a, &ex);    /* a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
        e = ex - 1;
        if (e < -6)
            e = -6;
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
    /* Now n in [8, 15] is a normal significand (1 + (n-8)/8) at exponent e, or e == -6 and
     * n in [0, 7] is a subnormal. Both map to code ((e + 7) << 3) + n - 8 for e >= -6 with the
     * subnormal case landing on e_field 0. */
    {
        int code;
        if (n < 8)
            code = (int)n;                              /* e == -6, subnormal or zero */
        else
            code = ((e + 7) << 3) + (int)(n - 8);
        /* a < 448 and the rounding above cannot pass 448 (the next step, 480, needs a >= 464). */
        return (uint8_t)(sign | code);
    }
}

void oracle_e4m3_encode_array(const float* v, uint8_t* codes, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        codes[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_encode_bits(uint32_t first, uint8_t* codes, int64_t n)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i;
        float f;
        memcpy(&f, &u, sizeof f);
        codes[i] = isnan(f) ? 0xFF : oracle_e4m3_encode(f);
    }
}

/* ---------------------------------------------------------------- one group */

/*
 * The per-group quantization step shared by all three groupings: the group's n valid values are
 * given in vals[]; their codes are written to codes[] and the stored (dequantization) scale is
 * returned.
 */
static float quantize_group(const float* vals, int64_t n, uint8_t* codes)
{
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
        codes[i] = oracle_e4m3_encode(v);
    }
    return s;
}

/* ---------------------------------------------------------------- quantizers */

int oracle_quantize_lhs(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* a_s)
{
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
            a_s[kb * M + m] = quantize_group(vals, n, codes);
            for (k = 0; k < n; ++k)
                q[m * ldq + k0 + k] = codes[k];
        }
    }
    return 0;
}

int oracle_quantize_rhs(const uint16_t* x, int64_t K, int64_t N, int64_t ldx,
                        uint8_t* qT, int64_t ldqT, float* s)
{
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
            s[kb * N + col] = quantize_group(vals, n, codes);
            for (k = 0; k < n; ++k)
                qT[col * ldqT + k0 + k] = codes[k];
        }
    }
    return 0;
}

int oracle_quantize_weight_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s)
{
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
        s[nb * Kb + kb] = quantize_group(vals, rn * rk, codes);
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
 * with A, B the decoded fp8 values. Products of two e4m3 values are exact in fp64 and a K-block's
 * partial sum of at most 128 of them is exact too (their magnitudes span under 2^45); only the
 * outer sum over K-blocks rounds, at fp64.
 * bscale_kind 0: 128x128 blocks via (stride_nb, stride_kb); 1: per column, b_s[kb * N + n].
 */
static int gemm_rows(const uint8_t* a, int64_t lda, const float* a_s,
                     const uint8_t* b, int64_t ldb, const float* b_s,
                     int bscale_kind, int64_t bs_stride_nb, int64_t bs_stride_kb,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t nrows, double* out)
{
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
        table[i] = oracle_e4m3_decode((uint8_t)i);

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
                              const int64_t* rows, int64_t nrows, double* out)
{
    return gemm_rows(a, lda, a_s, b, ldb, b_s, 0, bs_stride_nb, bs_stride_kb, M, N, K,
                     rows, nrows, out);
}

int oracle_gemm_1x128_128x1(const uint8_t* a, int64_t lda, const float* a_s,
                            const uint8_t* b, int64_t ldb, const float* b_s,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t* rows, int64_t nrows, double* out)
{
    return gemm_rows(a, lda, a_s, b, ldb, b_s, 1, 0, 0, M, N, K, rows, nrows, out);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
