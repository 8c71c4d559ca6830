/*
 * Blockwise-scaled FP8 oracle: plain CPU reference of the quantize + scaled-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the benchmark's CPU
 * baseline leg may load or call this library. The product path never links it and shares no code,
 * header, table or constant with it.
 *
 * Conventions (all host memory, caller-owned):
 *   bf16 tensors are uint16 bit patterns, row-major with a row stride in elements;
 *   fp8 tensors are uint8 codes, row-major with a row stride in bytes, in the format `fmt` names:
 *   ORACLE_FMT_E4M3FN (OCP float8_e4m3fn, finfo max 448) or ORACLE_FMT_E4M3FNUZ (float8_e4m3fnuz,
 *   finfo max 240);
 *   scales are fp32.
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef BSFP8_ORACLE_H
#define BSFP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_FMT_E4M3FN 0
#define ORACLE_FMT_E4M3FNUZ 1

/* Element codecs, written from the format definitions (round to nearest even, saturating). */
uint8_t oracle_e4m3_encode(float v);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3fnuz_encode(float v);
double oracle_e4m3fnuz_decode(uint8_t code);
void oracle_e4m3_encode_array(const float* v, uint8_t* codes, int64_t n);
/* Same, over every fp32 bit pattern in [first, first + n); for exhaustive sweeps. */
void oracle_e4m3_encode_bits(uint32_t first, uint8_t* codes, int64_t n);
/* Either format. */
void oracle_fp8_encode_array(int fmt, const float* v, uint8_t* codes, int64_t n);
void oracle_fp8_encode_bits(int fmt, uint32_t first, uint8_t* codes, int64_t n);

/* 1 x 128 row-wise groups of x [M, K]; a_s is column-major [M, ceil(K/128)] with ld = M. */
int oracle_quantize_lhs(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* a_s, int fmt);

/* 128 x 1 column-wise groups of x [K, N]; codes transposed to qT [N, K]; s row-major [ceil(K/128), N]. */
int oracle_quantize_rhs(const uint16_t* x, int64_t K, int64_t N, int64_t ldx,
                        uint8_t* qT, int64_t ldqT, float* s, int fmt);

/* 128 x 128 blocks of w [N, K]; q [N, K]; optional qT [K, N] (NULL to skip); s row-major [Nb, Kb]. */
int oracle_quantize_weight_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT, float* s,
                                   int fmt);

/*
 * Scaled GEMMs over fp8 codes, exact products and fp64 sums. Computes the full rows listed in
 * rows[0..nrows) of C [M, N] into out[r * N + n] (fp64, not rounded).
 *   a  [M, K] codes (lda), a_s column-major [M, Kb] (ld = M); a and b both in format fmt;
 *   b  [N, K] codes (ldb);
 *   128x128 variant: scale of (kb, n) is b_s[(n/128) * bs_stride_nb + kb * bs_stride_kb];
 *   128x1 variant:   scale of (kb, n) is b_s[kb * N + n].
 */
int oracle_gemm_1x128_128x128(const uint8_t* a, int64_t lda, const float* a_s,
                              const uint8_t* b, int64_t ldb, const float* b_s,
                              int64_t bs_stride_nb, int64_t bs_stride_kb,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t* rows, int64_t nrows, double* out, int fmt);
int oracle_gemm_1x128_128x1(const uint8_t* a, int64_t lda, const float* a_s,
                            const uint8_t* b, int64_t ldb, const float* b_s,
                            int64_t M, int64_t N, int64_t K,
                            const int64_t* rows, int64_t nrows, double* out, int fmt);

/* Threads the OpenMP loops above use. */
int oracle_num_threads(void);
/* Threads the parallel loops use from now on (n > 0). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
