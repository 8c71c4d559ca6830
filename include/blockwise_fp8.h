/*
 * blockwise_fp8.h: C ABI of the MI355X (gfx950) blockwise-scaled FP8 linear-layer kernels.
 *
 * The operations are those of pytorch/ao's blockwise FP8 training path as its pull-request pages
 * describe it:
 *   - "Enable blockwise FP8 dense training kernels on ROCm": description (FP8_MAX is the float8
 *     format's finfo max), quantization-correctness table (act_quant_lhs, act_quant_rhs,
 *     weight_quant_rhs, block_size 128), GEMM SQNR table, and the root-cause comment (the LHS
 *     quantizer stores reciprocal scales column-major; stores of rows >= M must be masked);
 *   - "Mask a_s/b_s scale loads in blockwise FP8 training GEMM kernels": Summary and Fix (the
 *     1x128_128x128 and 1x128_128x1 GEMMs; scale loads of rows >= M / columns >= N are masked).
 *
 * Element formats
 *   bf16   : 16-bit bfloat16 bit patterns (uint16).
 *   fp8    : OCP float8_e4m3fn codes (uint8): bias 7, largest finite 448, no infinities.
 *            The *_fnuz entry points use float8_e4m3fnuz codes instead (the format of the ROCm
 *            page's MI300X runs): bias 8, largest finite 0x7F = 240, no infinities, no negative
 *            zero (0x80 is its only NaN and is never produced). Their FP8_MAX is 240.
 *   scales : IEEE fp32.
 *
 * Quantization of one group g (1x128, 128x1 or 128x128 elements; a group at a tensor edge has only
 * its in-range elements):
 *   amax = max |x| over g;  amax_c = max(amax, 1e-12f);
 *   s    = amax_c / FP8_MAX  (IEEE fp32 division; the stored, dequantizing scale: x ~= dec(q) * s)
 *   m    = FP8_MAX / amax_c  (IEEE fp32 division)
 *   q    = enc( clamp(fl32(x * m), -FP8_MAX, FP8_MAX) )   round to nearest, ties to even;
 *   FP8_MAX = 448 (e4m3fn; the sign of a zero result is kept) or 240 (e4m3fnuz; zero is 0x00).
 *
 * Scaled GEMM (C = A B^T with both operands K-contiguous):
 *   C[m,n] = sum_kb  a_s[m,kb] * b_s(kb,n) * sum_{k in block kb, k < K} dec(A[m,k]) dec(B[n,k])
 *   Each K-block's inner sum is one 128-deep fp8 matrix-core dot product with fp32 output (measured
 *   on gfx950: not an exactly rounded fp32 sum; its error stays below about 2^-11 of the largest
 *   product in the block); it is multiplied by its two scales and added to an fp32 total before
 *   the next block; C is rounded to bf16 (RNE).
 *
 * Memory and ownership
 *   Every tensor pointer is a DEVICE pointer owned by the caller; the library retains none of
 *   them. Its state per device: the architecture check, the compute-unit count, and a
 *   stream-ordered memory pool for the K-split workspace of gemm_1x128_128x128 and
 *   gemm_1x128_128x1 (fp32 partial tiles, at most 256 MiB per call, allocated and freed on the
 *   call's stream around its two kernels; the pool keeps freed memory for reuse until the process
 *   ends). No other entry point allocates.
 *   Row-major tensors take a row stride "ld" in elements (bytes for fp8).
 *   Outputs must not overlap inputs. Every in-range output element is written; nothing outside the
 *   in-range elements (padding between rows, rows >= M, ...) is written.
 *
 * Calls are asynchronous: arguments are validated, kernels are enqueued on `stream` (a hipStream_t
 * passed as void*, NULL = the default stream) and the call returns. Results are ready once the
 * caller synchronizes the stream. Calls are thread-safe.
 *
 * Return codes
 *   BSFP8_OK (0); BSFP8_EINVAL (1) bad argument: a null pointer with a non-empty extent, a negative
 *   size, ld smaller than the row length, a stride out of range, a GEMM beyond its size limits;
 *   BSFP8_EALIGN (2) a GEMM operand
 *   row is not 16-byte aligned (see the GEMMs); BSFP8_EDEVICE (3) the current device is not gfx950;
 *   BSFP8_EHIP (4) a HIP call or launch failed; BSFP8_ESCRATCH (5) gemm_1x128_128x128_noalloc's
 *   split workspace would exceed its scratch. Argument checks happen before any HIP call, so
 *   codes 1 and 2 need no GPU. Empty problems (a zero extent) return BSFP8_OK without launching,
 *   except that a GEMM with K == 0 and M, N > 0 writes C = 0.
 */
#ifndef BLOCKWISE_FP8_H
#define BLOCKWISE_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BSFP8_OK = 0,
    BSFP8_EINVAL = 1,
    BSFP8_EALIGN = 2,
    BSFP8_EDEVICE = 3,
    BSFP8_EHIP = 4,
    BSFP8_ESCRATCH = 5
};

/* Text for a return code (static storage). */
const char* bsfp8_status_string(int status);

/*
 * quantize_lhs: 1x128 row-wise activation quantizer (act_quant_lhs).
 *   x   [M, K] bf16, row stride ldx >= K.
 *   q   [M, K] fp8, row stride ldq >= K.
 *   a_s column-major [M, ceil(K/128)] fp32 with leading dimension exactly M: the scale of row m,
 *       K-block kb is a_s[kb * M + m] (the layout of the ROCm page's root-cause comment; nothing
 *       past M * ceil(K/128) floats is written).
 * Any alignment and row length are accepted. With x and q 16-byte aligned, ldx % 8 == 0,
 * ldq % 16 == 0 and K % 16 == 0 each workgroup reads a strip of whole rows (or of up to 32
 * K-blocks of them) and then writes it; other 16-byte-aligned rows whose length is a multiple of 8
 * take the vector tile path, the rest load and store element by element. The result is the same
 * on every path. The environment variable BSFP8_QUANT_LHS_STRIP (1, 2, 4, 8, 16: strips of that
 * many 16-byte pieces per thread; 0: tiles), read at each call, overrides the choice for tests
 * and sweeps.
 */
int quantize_lhs(const void* x, int64_t M, int64_t K, int64_t ldx,
                 void* q, int64_t ldq, float* a_s, void* stream);

/*
 * quantize_rhs: 128x1 column-wise activation quantizer (act_quant_rhs), with transposed output.
 *   x   [K, N] bf16 row-major, row stride ldx >= N; groups are 128 consecutive rows of a column.
 *   qT  [N, K] fp8 row-major (K-contiguous), row stride ldqT >= K: qT[n, k] is the code of x[k, n].
 *   s   [ceil(K/128), N] fp32 row-major: s[kb * N + n]. These bytes equal a column-major
 *       [N, ceil(K/128)] a_s with ld N, so qT/s can be the A operand of either GEMM.
 */
int quantize_rhs(const void* x, int64_t K, int64_t N, int64_t ldx,
                 void* qT, int64_t ldqT, float* s, void* stream);

/*
 * quantize_weight_128x128: 128x128 block weight quantizer (weight_quant_rhs).
 *   w   [N, K] bf16 (nn.Linear layout [out, in]), row stride ldw >= K.
 *   q   [N, K] fp8, row stride ldq >= K.
 *   qT  [K, N] fp8 or NULL: the same codes transposed (the dgrad operand), row stride ldqT >= N.
 *   s   [ceil(N/128), ceil(K/128)] fp32 row-major: s[nb * ceil(K/128) + kb].
 */
int quantize_weight_128x128(const void* w, int64_t N, int64_t K, int64_t ldw,
                            void* q, int64_t ldq, void* qT, int64_t ldqT,
                            float* s, void* stream);

/*
 * quantize_lhs_and_rhs: both activation quantizations of one tensor in a single pass (the input is
 * read once), for a tensor that is the A operand of one GEMM and, transposed, an operand of the
 * weight-gradient GEMM (activations X and output gradients dY of a linear layer in training).
 *   x   [R, C] bf16, row stride ldx >= C.
 *   q, a_s  exactly what quantize_lhs(x, M = R, K = C) writes: q [R, C] fp8 (ldq >= C), a_s
 *           column-major [R, ceil(C/128)] with ld R.
 *   qT, s   exactly what quantize_rhs(x, K = R, N = C) writes: qT [C, R] fp8 (ldqT >= R), s
 *           [ceil(R/128), C] row-major.
 * The codes and scales are bit-identical to those two calls (act_quant_lhs and act_quant_rhs of the
 * ROCm page's quantization-correctness table); only the traffic differs: 2 B read and 2 B written
 * per element instead of 4 B and 2 B.
 */
int quantize_lhs_and_rhs(const void* x, int64_t R, int64_t C, int64_t ldx,
                         void* q, int64_t ldq, float* a_s,
                         void* qT, int64_t ldqT, float* s, void* stream);

/*
 * gemm_1x128_128x128: C = A B^T with 1x128 scales on A and 128x128 block scales on B
 * (forward Y = X W^T, and dgrad dX = dY W using the transposed weight codes).
 *   a   [M, K] fp8, row stride lda; a_s column-major [M, ceil(K/128)], ld M.
 *   b   [N, K] fp8, row stride ldb.
 *   b_s scale of (K-block kb, N-block nb) at b_s[nb * bs_stride_nb + kb * bs_stride_kb]
 *       (forward with the weight scales [Nb, Kb]: strides (Kb, 1); dgrad with the same weight
 *       scales read transposed: strides (1, Nb_of_weight)). Strides must be >= 0.
 *   c   [M, N] bf16, row stride ldc >= N.
 * Alignment (else BSFP8_EALIGN): a and b 16-byte aligned, lda and ldb multiples of 16.
 * Size limits (else BSFP8_EINVAL; every operand and scale read goes through a buffer resource of
 * at most 2^31 bytes, and a lane whose row, column or K-block is out of range is given an offset
 * past that resource's end, which the hardware reads as zero):
 *   256 * lda, 256 * ldb, 4 * M * ceil(K/128) and 4 * (the b_s elements the strides span) at most
 *   2^31; ceil(M/128) at most 65535.
 * Scale reads are limited to rows < M, columns < N and K-blocks < ceil(K/128).
 * Schedule: one workgroup per 256 x 256 output tile, or per 128 x 256 tile when M <= 128 or the
 * 256-row tiles number at most half the compute units. When the 128 x 256 tiles would fill at most
 * half the compute units, one workgroup per 64 x 128, 64 x 64 or 64 x 32 tile (the widest whose
 * workgroups occupy three quarters of the compute units) over the whole K range; all tile shapes give
 * bit-identical results. Only when
 * those tiles are fewer than half the compute units and K exceeds 64 blocks are the K-blocks split
 * over S workgroups per 128- or 256-row tile, which write fp32 partial tiles to the pooled
 * workspace, and a second kernel sums the S partials in a fixed order into C (same result on every
 * call). When the 256 x 256 tiles end in a last round that would fill at most a quarter of the
 * compute units and K is long enough, the leading columns that fill whole rounds run as one GEMM and
 * the remaining columns as a second with K split in at least four (128 x 128 B scales only; the
 * leading columns' results are those of the unsplit schedule bit for bit; BSFP8_GEMM_COLUMN_SPLIT=0
 * turns it off). The environment variables BSFP8_GEMM_SPLIT, BSFP8_GEMM_TILE_M, BSFP8_GEMM_TILE_N,
 * BSFP8_GEMM_THIN_STAGES and BSFP8_GEMM_THIN_WAVES, read at each call, force S (1 = never split; S
 * is clamped to ceil(K/128) and to the workspace bound; a split uses the 128- or 256-row tiles), the
 * tile height (256, 128 or 64), the width of the 64-row tiles (32, 64 or 128), their LDS pipeline
 * depth (2, 3, 4, 6, 8 or 12 where the tile's stages fit) and their waves per workgroup (4, or 8 for
 * 64- and 128-column tiles); a depth or wave count outside these is BSFP8_EHIP before any launch.
 */
int gemm_1x128_128x128(const void* a, int64_t lda, const float* a_s,
                       const void* b, int64_t ldb, const float* b_s,
                       int64_t bs_stride_nb, int64_t bs_stride_kb,
                       void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_1x128_128x128_noalloc: gemm_1x128_128x128 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, result, limits and split schedule; the K-split partial tiles live in a static scratch
 * array of 64 MiB that each GPU holds for the life of the process, so the call allocates nothing
 * (no hipMalloc, no pool). 64 MiB covers every automatic split plan; a plan forced larger through
 * BSFP8_GEMM_SPLIT returns BSFP8_ESCRATCH before any launch. The column split of a partial last
 * round runs here only when its tail's partial tiles fit the scratch; otherwise this entry runs the
 * unsplit schedule, whose tail columns can then differ from gemm_1x128_128x128's in the last bits. Every call on one GPU shares that
 * GPU's scratch: calls on one stream are ordered, but calls that overlap in time on one GPU (other
 * streams, other threads) race on it. No part of the scratch needs clearing (each slice writes its
 * whole partial tile before the sum reads it).
 */
int gemm_1x128_128x128_noalloc(const void* a, int64_t lda, const float* a_s,
                               const void* b, int64_t ldb, const float* b_s,
                               int64_t bs_stride_nb, int64_t bs_stride_kb,
                               void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_1x128_128x1: C = A B^T with 1x128 scales on A and per-column 128x1 scales on B
 * (wgrad dW = dY^T X, contracting over tokens: A and B are quantize_rhs outputs).
 *   a, lda, a_s as above;  b [N, K] fp8, row stride ldb;
 *   b_s [ceil(K/128), N] fp32 row-major: the scale of (kb, n) is b_s[kb * N + n].
 *   c   [M, N] bf16, row stride ldc >= N.  Alignment, size limits and schedule as for
 *   gemm_1x128_128x128 (4 * N * ceil(K/128) at most 2^31 in place of the b_s span).
 */
int gemm_1x128_128x1(const void* a, int64_t lda, const float* a_s,
                     const void* b, int64_t ldb, const float* b_s,
                     void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_1x128_128x128_grouped: the forward (or dgrad) GEMM of an expert-grouped (mixture-of-experts)
 * layer in one launch. Tokens are sorted by expert: expert e owns rows [offsets[e], offsets[e+1])
 * of A and C and multiplies them by its own B_e with its own 128x128 scales -- the grouped form of
 * gemm_1x128_128x128 (the MoE path the ROCm page's description refers to, whose kernels it does not
 * list; this is the plainest reading: per expert, exactly gemm_1x128_128x128 on its rows).
 *   a, lda, a_s   all tokens: A [M, K] fp8, a_s column-major [M, ceil(K/128)] with ld M (one
 *                 quantize_lhs over all tokens: 1x128 groups lie inside a token row).
 *   b, ldb        B_e = b + e * b_stride (bytes), [N, K] rows of stride ldb. For stacked weights
 *                 W [E, N, K] quantized as one [E*N, K] matrix (N % 128 == 0): forward b = q,
 *                 b_stride = N * ldq; dgrad b = its transposed codes qT [K, E*N], b_stride = N bytes,
 *                 ldb = ldqT.
 *   b_s           scales of B_e at b_s + e * bs_stride (floats), (K-block kb, N-block nb) at
 *                 [nb * bs_stride_nb + kb * bs_stride_kb], as in gemm_1x128_128x128.
 *   offsets       E + 1 int64 in DEVICE memory, non-decreasing, in [0, M]. The kernel clamps them
 *                 into [0, M] and to non-decreasing order; rows outside every range are not written.
 *   c, ldc        C [M, N] bf16.
 * Requirements (else BSFP8_EINVAL): K a positive multiple of 128; b_stride a multiple of 16 (else
 * BSFP8_EALIGN); alignment and size limits as gemm_1x128_128x128. Never split; allocates nothing.
 * E == 0 or an empty M or N: no launch.
 */
int gemm_1x128_128x128_grouped(const void* a, int64_t lda, const float* a_s,
                               const void* b, int64_t ldb, int64_t b_stride,
                               const float* b_s, int64_t bs_stride,
                               int64_t bs_stride_nb, int64_t bs_stride_kb,
                               const int64_t* offsets, int64_t E,
                               void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_1x128_128x1_grouped: the weight gradient of an expert-grouped layer in one launch: for every
 * expert e, C_e = A_e B_e^T where A_e and B_e are the columns (tokens) [offsets[e], offsets[e+1])
 * of A and B -- per expert, exactly gemm_1x128_128x1 over its own tokens.
 *   a, lda, a_s   A [M, K] fp8 = the 128x1 codes of dY over all K token columns, a_s [K/128, M].
 *   b, ldb, b_s   B [N, K] fp8 = the 128x1 codes of X, b_s [K/128, N].
 *   offsets       E + 1 int64 token boundaries in DEVICE memory, clamped into [0, K] and to
 *                 non-decreasing order. Each expert's 128x1 groups must lie inside its own tokens:
 *                 every boundary a multiple of 128. That holds for quantize_rhs_grouped's padded
 *                 boundaries (any routing), or for quantize_rhs over all tokens when the experts'
 *                 token counts are multiples of 128.
 *   c, ldc        E outputs [M, N] bf16, expert e's at c + e * c_stride (elements).
 *   status        NULL or a DEVICE int32: an expert whose clamped boundaries are not multiples of
 *                 128 is not computed -- its C_e is filled with NaN -- and *status is set to 1
 *                 (the kernel never clears it). Nothing is rounded to the 128 grid.
 * Requirements (else BSFP8_EINVAL): K a positive multiple of 128, E <= 65535,
 * c_stride >= (M - 1) * ldc + N when E > 1; alignment and size limits as gemm_1x128_128x1.
 * Never split; allocates nothing.
 */
int gemm_1x128_128x1_grouped(const void* a, int64_t lda, const float* a_s,
                             const void* b, int64_t ldb, const float* b_s,
                             const int64_t* offsets, int64_t E,
                             void* c, int64_t ldc, int64_t c_stride,
                             int64_t M, int64_t N, int64_t K, int32_t* status, void* stream);

/*
 * quantize_rhs_grouped: 128x1 column-wise quantization (act_quant_rhs) of expert-grouped tokens whose
 * groups restart at every expert's first token -- the per-expert quantize_rhs the MoE weight
 * gradient needs when routing gives token counts that are not multiples of 128 (the MoE path the
 * ROCm page's description refers to; this is the plainest reading: per expert, exactly quantize_rhs
 * of its own tokens).
 *   x        [T, N] bf16, row stride ldx >= N; expert e owns rows [offsets[e], offsets[e+1]).
 *   offsets  E + 1 int64 in DEVICE memory, clamped into [0, T] and to non-decreasing order.
 *   Output in the 128-padded token layout: P[e] = sum over the experts before e of their token
 *   counts rounded up to a multiple of 128.
 *   qT       [N, ldqT] fp8 (transposed codes), ldqT >= 128 G with G = ceil(T/128) + E: column
 *            P[e] + t holds expert e's token t, the columns up to the next multiple of 128 hold 0;
 *            columns from P[E] on are not written.
 *   s        fp32 [G, N] row-major: row p holds the scales of padded group p (columns 128 p ..
 *            128 p + 127 of qT); rows from P[E] / 128 on are not written. An expert's last group
 *            takes its amax over the tokens it has.
 *   padded_offsets  E + 1 int64 in DEVICE memory, written with P (P[0] = 0, P[E] the padded total).
 * Pass qT, s and padded_offsets to gemm_1x128_128x1_grouped with K = 128 G. Requirements (else
 * BSFP8_EINVAL): G <= 65535, offsets and padded_offsets not NULL.
 */
int quantize_rhs_grouped(const void* x, int64_t T, int64_t N, int64_t ldx,
                         const int64_t* offsets, int64_t E,
                         void* qT, int64_t ldqT, float* s, int64_t* padded_offsets, void* stream);

/*
 * encode_e4m3_f32: the quantizers' element conversion applied to n arbitrary fp32 values:
 *   q[i] = e4m3(clamp(x[i], -448, 448)), round to nearest even, sign kept. NaN inputs are outside
 *   the contract. Exposed so the device conversion can be checked over every fp32 pattern.
 *   Alignment (else BSFP8_EALIGN): x 16-byte aligned, q 4-byte aligned.
 */
int encode_e4m3_f32(const float* x, void* q, int64_t n, void* stream);

/*
 * quantize_lhs_and_weight: quantize_lhs(x) and quantize_weight_128x128(w) in one launch -- the two
 * quantizations of a linear layer's forward step (Y = X W^T: the 1x128 groups of the activation
 * and the 128x128 blocks of the weight, "Enable blockwise FP8 dense training kernels on ROCm",
 * quantization-correctness table). The outputs are byte-identical to the two separate calls with
 * the same arguments:
 *   x [M, K] bf16 (ldx), qx [M, K] (ldqx), sx column-major [M, ceil(K/128)] with ld M;
 *   w [N, Kw] bf16 (ldw), qw [N, Kw] (ldqw), qwT nullable [Kw, N] (ldqwT), sw [Nb, Kbw] row-major.
 * Either tensor may be empty (then only the other one is quantized). With 16-byte bf16 rows,
 * 8-byte code rows and 16-byte qwT rows both run in one persistent kernel; otherwise the two
 * single-purpose kernels run one after the other. Errors as for the two calls.
 */
int quantize_lhs_and_weight(const void* x, int64_t M, int64_t K, int64_t ldx,
                            void* qx, int64_t ldqx, float* sx,
                            const void* w, int64_t N, int64_t Kw, int64_t ldw,
                            void* qw, int64_t ldqw, void* qwT, int64_t ldqwT, float* sw,
                            void* stream);

/*
 * float8_e4m3fnuz variants ("Enable blockwise FP8 dense training kernels on ROCm", description:
 * FP8_MAX follows torch.finfo(dtype) and both float8_e4m3fn and float8_e4m3fnuz are accepted; its
 * MI300X log runs e4m3fnuz with FP8 max 240). Each takes exactly the arguments of the entry point
 * it is named after, with the same layouts, limits, alignment rules and return codes; the codes
 * it writes or reads are e4m3fnuz and FP8_MAX is 240.
 *   Quantizers: the same kernels as the e4m3fn ones.
 *   GEMMs: gfx950's FP8 matrix instructions read e4m3fn only, and e4m3fnuz values (2^-10 .. 240)
 *     are not all e4m3fn values under any one power-of-two scaling, so these widen each code
 *     exactly to f16 in registers and run the K-block as four 16x16x32 f16 matrix instructions
 *     (fp32 accumulation, the same per-K-block rescale and bf16 rounding). Both operands must be
 *     e4m3fnuz; the expert-grouped GEMMs have no e4m3fnuz variant.
 *   encode_e4m3fnuz_f32: q[i] = e4m3fnuz(x[i]) by the quantizers' conversion, for
 *     |x[i]| <= 240 (1 + 2^-21) -- the range a group multiplier produces; larger magnitudes are
 *     outside the contract. Exposed so the device conversion can be checked exhaustively.
 */
int quantize_lhs_fnuz(const void* x, int64_t M, int64_t K, int64_t ldx,
                      void* q, int64_t ldq, float* a_s, void* stream);
int quantize_rhs_fnuz(const void* x, int64_t K, int64_t N, int64_t ldx,
                      void* qT, int64_t ldqT, float* s, void* stream);
int quantize_weight_128x128_fnuz(const void* w, int64_t N, int64_t K, int64_t ldw,
                                 void* q, int64_t ldq, void* qT, int64_t ldqT, float* s,
                                 void* stream);
int quantize_lhs_and_rhs_fnuz(const void* x, int64_t R, int64_t C, int64_t ldx,
                              void* q, int64_t ldq, float* a_s,
                              void* qT, int64_t ldqT, float* s, void* stream);
int quantize_lhs_and_weight_fnuz(const void* x, int64_t M, int64_t K, int64_t ldx,
                                 void* qx, int64_t ldqx, float* sx,
                                 const void* w, int64_t N, int64_t Kw, int64_t ldw,
                                 void* qw, int64_t ldqw, void* qwT, int64_t ldqwT, float* sw,
                                 void* stream);
int gemm_1x128_128x128_fnuz(const void* a, int64_t lda, const float* a_s,
                            const void* b, int64_t ldb,
                            const float* b_s, int64_t bs_stride_nb, int64_t bs_stride_kb,
                            void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);
int gemm_1x128_128x1_fnuz(const void* a, int64_t lda, const float* a_s,
                          const void* b, int64_t ldb, const float* b_s,
                          void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);
int encode_e4m3fnuz_f32(const float* x, void* q, int64_t n, void* stream);
int quantize_rhs_grouped_fnuz(const void* x, int64_t T, int64_t N, int64_t ldx,
                              const int64_t* offsets, int64_t E,
                              void* qT, int64_t ldqT, float* s, int64_t* padded_offsets, void* stream);

#ifdef __cplusplus
}
#endif
#endif
