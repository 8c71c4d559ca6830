// gfx950 blockwise-scaled FP8 GEMM: C[M,N] (bf16) = A[M,K] . B[N,K]^T with a 1x128 scale per
// (row, K-block) on A and either a 128x128 block scale or a 128x1 per-column scale on B
// (triton_fp8_gemm_1x128_128x128 / _128x1 of "Mask a_s/b_s scale loads in blockwise FP8 training
// GEMM kernels", Summary; the scale loads there are masked to rows < M and columns < N, as every
// scale load here is).
//
// Tile engine
//   * one K-block (128) is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output subtile, so a
//     K-block's partial sum comes out of the matrix core in one instruction with zero C-in;
//   * the partial is multiplied by a_s[m,kb] * b_s(kb,n) and added into fp32 totals (one FMA per
//     element per K-block) before the next K-block, as the method prescribes;
//   * the MFMA is issued with B as its first operand, so a lane's four outputs are four consecutive
//     columns n of one row m: the 128x128 rescale factor is one scalar per (lane, M-subtile) and
//     the bf16 epilogue writes 8 contiguous bytes per lane;
//   * A and B tiles are staged in LDS with a 16-byte-chunk XOR swizzle (chunk ^ row%8) so the
//     fragment reads (16 rows x 32 bytes per 16 lanes) are bank-conflict free;
//   * rows >= M / columns >= N are never loaded (zero in LDS) nor stored; a ragged last K-block is
//     zero-filled beyond K.
#include "device_common.hpp"
#include "launch.hpp"

namespace bsfp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // Format selectors 0/0 = float8_e4m3fn for both operands; scale operands 0 select the
    // unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
}

// 16 bytes of an fp8 row starting at column kc; columns >= K are zero. Rows are 16-byte aligned.
__device__ __forceinline__ uint4 load16_k(const uint8_t* __restrict__ row, int64_t kc, int64_t K) {
    if (kc + 16 <= K) return *reinterpret_cast<const uint4*>(row + kc);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16; ++j)
        if (kc + j < K) w[j >> 2] |= static_cast<uint32_t>(row[kc + j]) << (8 * (j & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool PER_COL>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ b_s,
    int64_t bs_nb, int64_t bs_kb, uint16_t* __restrict__ C, int64_t ldc,
    int64_t M, int64_t N, int64_t K, int c_vec) {
    __shared__ uint4 sA[kBM * 8];
    __shared__ uint4 sB[kBN * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
    const int64_t Kb = (K + kGroup - 1) / kGroup;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t kb = 0; kb < Kb; ++kb) {
        const int64_t k0 = kb * kGroup;
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = (tid >> 3) + 32 * p;
            const int ch = tid & 7;
            const int64_t kc = k0 + ch * 16;
            uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = make_uint4(0u, 0u, 0u, 0u);
            if (m0 + r < M) va = load16_k(A + (m0 + r) * lda, kc, K);
            if (n0 + r < N) vb = load16_k(B + (n0 + r) * ldb, kc, K);
            sA[r * 8 + (ch ^ (r & 7))] = va;
            sB[r * 8 + (ch ^ (r & 7))] = vb;
        }
        __syncthreads();

        v8i af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + i * 16 + l16;
            const uint4 lo = sA[r * 8 + ((2 * lg) ^ (r & 7))];
            const uint4 hi = sA[r * 8 + ((2 * lg + 1) ^ (r & 7))];
            af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 64 + j * 16 + l16;
            const uint4 lo = sB[r * 8 + ((2 * lg) ^ (r & 7))];
            const uint4 hi = sB[r * 8 + ((2 * lg + 1) ^ (r & 7))];
            bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }

        // scales: the lane's row m of each M-subtile; masked to m < M
        float as[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + wm * 64 + i * 16 + l16;
            as[i] = (m < M) ? a_s[kb * M + m] : 0.0f;
        }
        if (!PER_COL) {
            const float bsc = b_s[static_cast<int64_t>(blockIdx.x) * bs_nb + kb * bs_kb];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = as[i] * bsc;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f p = mfma_fp8_16x16x128(bfr[j], af[i]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r], f, acc[i][j][r]);
                }
            }
        } else {
            float bsv[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + wn * 64 + j * 16 + 4 * lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) bsv[j][r] = (n + r < N) ? b_s[kb * N + n + r] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f p = mfma_fp8_16x16x128(bfr[j], af[i]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][r] = fmaf(p[r], as[i] * bsv[j][r], acc[i][j][r]);
                }
            }
        }
    }

    // epilogue: lane holds C[m][n .. n+3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 64 + i * 16 + l16;
        if (m >= M) continue;
        uint16_t* crow = C + m * ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + j * 16 + 4 * lg;
            const uint32_t w0 = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t w1 = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            if (c_vec && n + 4 <= N) {
                *reinterpret_cast<uint2*>(crow + n) = make_uint2(w0, w1);
            } else {
                const uint16_t h[4] = {static_cast<uint16_t>(w0 & 0xFFFF), static_cast<uint16_t>(w0 >> 16),
                                       static_cast<uint16_t>(w1 & 0xFFFF), static_cast<uint16_t>(w1 >> 16)};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) crow[n + r] = h[r];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                       int64_t ldb, BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((N + kBN - 1) / kBN), static_cast<unsigned>((M + kBM - 1) / kBM));
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 8 == 0) && (ldc % 4 == 0);
    if (bs.per_column)
        gemm_kernel<true><<<grid, kThreads, 0, stream>>>(a, lda, a_s, b, ldb, bs.ptr, 0, 0, c, ldc,
                                                         M, N, K, c_vec);
    else
        gemm_kernel<false><<<grid, kThreads, 0, stream>>>(a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb,
                                                          bs.stride_kb, c, ldc, M, N, K, c_vec);
    return hipGetLastError();
}

}  // namespace bsfp8
