// gfx950 blockwise-scaled FP8 GEMM: C[M,N] (bf16) = A[M,K] . B[N,K]^T with a 1x128 scale per
// (row, K-block) on A and either a 128x128 block scale or a 128x1 per-column scale on B
// (triton_fp8_gemm_1x128_128x128 / _128x1 of "Mask a_s/b_s scale loads in blockwise FP8 training
// GEMM kernels", Summary; the scale loads there are masked to rows < M and columns < N, as every
// scale load here is).
//
// Shared by both kernels below:
//   * one K-block (128) is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output subtile, so a
//     K-block's partial sum comes out of the matrix core in one instruction with zero C-in;
//   * the partial is multiplied by a_s[m,kb] * b_s(kb,n) and added into fp32 totals (one FMA per
//     element per K-block) before the next K-block, as the method prescribes;
//   * the MFMA takes B as its first operand, so a lane's four outputs are four consecutive columns n
//     of one row m: the 128x128 rescale factor is one scalar per (lane, 16-row subtile) and the bf16
//     epilogue writes 8 contiguous bytes per lane;
//   * the fast kernel stages tiles in LDS with a 16-byte-chunk XOR swizzle and reads its fragments
//     bank-conflict free (its layout is described there);
//   * operands are read through buffer resources that end at the matrix edge: rows >= M / >= N read
//     as zero, and their outputs are never stored; every scale read is limited to rows < M,
//     columns < N.
// The fast kernel (namespace fast) serves every float8_e4m3fn GEMM whose B scales it can stage
// (per-column: N % 4 == 0; 128x128: at most 512 K-blocks), a partial last K-block included; the
// general kernel serves the rest and the float8_e4m3fnuz operands. Both zero the bytes of a
// partial last K-block that lie at or past K.
//
// float8_e4m3fnuz operands (the format of the ROCm page's MI300X runs, FP8_MAX 240) run on the
// general kernel: gfx950's FP8 matrix instructions read e4m3fn, and no power-of-two rescaling
// maps every fnuz value onto an e4m3fn value (fnuz spans 2^-10 .. 240, e4m3fn 2^-9 .. 448, and
// 2 x 240 = 480 is not an e4m3fn value). Each fnuz code is instead widened exactly to f16 in
// registers (its 7 magnitude bits placed under the f16 exponent field: the value times 2^-7, the
// smallest ones as f16 subnormals) and a K-block is four v_mfma_f32_16x16x32_f16 instead of one
// FP8 instruction -- products of two 4-significant-bit values are exact in fp32 either way, so the
// per-K-block partials equal the fn path's arithmetic up to the exact factor 2^-14.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace bsfp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef short s2v __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;      // workgroup rows (M)
constexpr int kBN = 128;      // workgroup columns (N)
constexpr int kWM = 64;       // rows per wave
constexpr int kWN = 64;       // columns per wave
constexpr int kWavesM = kBM / kWM;  // 4
constexpr int kWavesN = kBN / kWN;  // 2
constexpr int kThreads = 64 * kWavesM * kWavesN;  // 512: two waves per SIMD
constexpr int kMSub = kWM / 16;   // 16-row subtiles per wave
constexpr int kNSub = kWN / 16;   // 16-column subtiles per wave

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // Format selectors 0/0 = float8_e4m3fn for both operands; scale operands 0 select the
    // unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Two float8_e4m3fnuz codes (bytes 0,1 of w for HALF 0, bytes 2,3 for HALF 1) as two exact f16
// values scaled by 2^-7. Each code c = s eeee mmm is moved to bits 15..8 of its 16-bit half; an
// arithmetic shift by one leaves s in bit 15 (and a copy in bit 14, cleared next), e in the low four
// bits of the f16 exponent field and m at the top of the f16 mantissa. That f16 is
// (1 + m/8) 2^(e - 15), or (m/8) 2^-14 for e = 0 (an f16 subnormal), i.e. exactly the fnuz value
// times 2^-7. The matrix instructions take f16 subnormal inputs exactly (every code's value comes
// back exact through the GEMM), so the 2^14 of a product is folded into the per-K-block factor.
template <int HALF>
__device__ __forceinline__ uint32_t fnuz2_to_f16x2(uint32_t w) {
    const uint32_t p = __builtin_amdgcn_perm(w, w, HALF ? 0x030C020Cu : 0x010C000Cu);
    s2v v = __builtin_bit_cast(s2v, p);
    v = v >> 1;
    return __builtin_bit_cast(uint32_t, v) & 0xBFFFBFFFu;
}

// A 32-code FP8 fragment (the lane's operand of one 16x16x128 instruction) as the operands of four
// 16x16x32 f16 instructions: instruction q takes the lane's codes 8q .. 8q + 7. The lane-to-k
// assignment is the same for both operands, so the four instructions together sum over exactly the
// K-block's 128 products.
__device__ __forceinline__ void fnuz_frag_to_f16(const v8i& f, h8v (&out)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = static_cast<uint32_t>(f[2 * q]);
        const uint32_t w1 = static_cast<uint32_t>(f[2 * q + 1]);
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 h = {fnuz2_to_f16x2<0>(w0), fnuz2_to_f16x2<1>(w0), fnuz2_to_f16x2<0>(w1), fnuz2_to_f16x2<1>(w1)};
        out[q] = __builtin_bit_cast(h8v, h);
    }
}

__device__ __forceinline__ v4f mfma_f16_kblock(const h8v (&b)[4], const h8v (&a)[4]) {
    v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[q], a[q], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
}

template <int V>
struct IntTag {
    static constexpr int value = V;
};

// Workgroup -> output tile. Workgroups are dispatched round-robin over the 8 XCDs; consecutive
// logical tiles are given to the same XCD, and logical tiles are ordered in groups of kGroupRows
// tile-rows so the workgroups one XCD runs at the same time share A rows and B columns in its L2.
constexpr int kXcds = 8;
constexpr int kGroupRows = 4;

__device__ __forceinline__ void tile_of(int bid, int mt, int nt, int& tm, int& tn) {
    const int total = mt * nt;
    int logical = bid;
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    const int per_group = kGroupRows * nt;
    const int group = logical / per_group;
    const int first_m = group * kGroupRows;
    const int gsize = min(mt - first_m, kGroupRows);
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, static_cast<int>(bytes),
                                             0x00020000);
}

constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer this kernel builds

// Zero the bytes of a 16-byte chunk that lie at or past `valid` (valid counted from the chunk start).
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int64_t valid) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int64_t keep = valid - 4 * d;  // bytes of dword d to keep
        const uint32_t msk = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
        v[d] &= msk;
    }
    return v;
}

__device__ __forceinline__ v8i to_v8i(u32x4 lo, u32x4 hi) {
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Per-workgroup addressing state. Tensors are read through buffer resources whose extent stops at
// the last row of the matrix, so rows >= M (A) or >= N (B) read as zero; per-lane offsets are
// 32-bit and block/subtile steps are uniform (scalar) offsets.
struct Operands {
    __amdgpu_buffer_rsrc_t a, b, as, bs;
    uint32_t a_lane;          // (wave rows + l16) * lda + 32 lg  within the A tile
    uint32_t b_lane;          // (tid / 8) * ldb + 16 (tid % 8)   within the B tile
    uint32_t b_dma_lane;      // direct-to-LDS B load: row 16 wave + lane / 8, chunk (lane % 8) ^ (lane / 8)
    uint32_t as_off[kMSub];   // 4 * m, or kOob for m >= M
    uint32_t bs_off[kNSub];   // 4 * n for the per-column scales (n = first of the lane's 4), or kOob
    uint32_t bs_partial;      // bit j: the lane's 4 columns of subtile j straddle column N
    uint32_t a_sub;           // 16 * lda: A offset between consecutive 16-row subtiles
    uint32_t b_half;          // 64 * ldb: B offset between the 2 row halves a thread loads
    uint32_t b_eighth;        // 8 * ldb
};

// A operand of K-block kb for this lane: subtile i covers rows 16 i + l16 of the wave's 64 rows and
// bytes [32 lg, 32 lg + 32) of the block, exactly the MFMA's per-lane operand layout.
template <bool FULL>
__device__ __forceinline__ void load_a(v8i (&af)[kMSub], const Operands& op, int64_t kb, int64_t K, int lg) {
#pragma unroll
    for (int i = 0; i < kMSub; ++i) {
        const uint32_t so = static_cast<uint32_t>(i) * op.a_sub + static_cast<uint32_t>(kb * kGroup);
        u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(op.a, op.a_lane, so, 0);
        u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(op.a, op.a_lane + 16, so, 0);
        if (!FULL) {
            const int64_t valid = K - (kb * kGroup + 32 * lg);
            lo = mask_tail(lo, valid);
            hi = mask_tail(hi, valid - 16);
        }
        af[i] = to_v8i(lo, hi);
    }
}

// B tile of K-block kb (128 rows x 128 bytes) into registers: thread t holds rows t/8 + 64 p,
// 16-byte chunk t % 8.
template <bool FULL>
__device__ __forceinline__ void load_b(u32x4 (&bst)[2], const Operands& op, int64_t kb, int64_t K, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const uint32_t so = static_cast<uint32_t>(p) * op.b_half + static_cast<uint32_t>(kb * kGroup);
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(op.b, op.b_lane, so, 0);
        if (!FULL) v = mask_tail(v, K - (kb * kGroup + 16 * (tid & 7)));
        bst[p] = v;
    }
}

// LDS image of a B tile: row r, 16-byte chunk c stored at chunk position c ^ (r % 8), so the
// fragment reads (rows 16 j .. 16 j + 15 at one logical chunk) spread over all banks.
__device__ __forceinline__ void store_b(u32x4* __restrict__ sb, const u32x4 (&bst)[2], int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = (tid >> 3) + 64 * p;
        const int ch = tid & 7;
        sb[r * 8 + (ch ^ (r & 7))] = bst[p];
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// B tile of a full K-block straight from global memory into its LDS image (no registers): wave w
// fills tile rows [16 w, 16 w + 16) with two 1 KB loads; lane i of load q lands at 16-byte position
// (16 w + 8 q) * 8 + i, i.e. row 16 w + 8 q + i / 8, chunk position i % 8, which holds logical chunk
// (i % 8) ^ (i / 8) of that row -- the same swizzled image store_b writes.
__device__ __forceinline__ void dma_b(u32x4* __restrict__ sb, const Operands& op, int64_t kb, int wave) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        lds_void_t* dst = (lds_void_t*)(sb + (16 * wave + 8 * q) * 8);
        const uint32_t so = static_cast<uint32_t>(q) * op.b_eighth + static_cast<uint32_t>(kb * kGroup);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op.b, dst, 16, op.b_dma_lane, so, 0, 0);
    }
}

template <bool PER_COL>
__device__ __forceinline__ void load_scales(float (&as)[kMSub], u32x4 (&bsv)[kNSub], float& bscal,
                                            const Operands& op, const float* __restrict__ b_s,
                                            int64_t bs_nb, int64_t bs_kb, int64_t kb, int64_t M,
                                            int64_t N, int tn) {
    const uint32_t col = static_cast<uint32_t>(kb * M * 4);
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
        as[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(op.as, op.as_off[i], col, 0));
    if (PER_COL) {
        const uint32_t row = static_cast<uint32_t>(kb * N * 4);
#pragma unroll
        for (int j = 0; j < kNSub; ++j) {
            if (op.bs_partial & (1u << j)) {  // the quad straddles column N: per-element loads
                const int64_t n = op.bs_off[j] / 4;
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (n + e < N) ? __builtin_amdgcn_raw_buffer_load_b32(op.bs, op.bs_off[j] + 4 * e, row, 0) : 0u;
                bsv[j] = v;
            } else {
                bsv[j] = __builtin_amdgcn_raw_buffer_load_b128(op.bs, op.bs_off[j], row, 0);
            }
        }
    } else {
        bscal = b_s[static_cast<int64_t>(tn) * bs_nb + kb * bs_kb];
    }
}

template <bool PER_COL, bool FNUZ>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ b_s,
    int64_t bs_nb, int64_t bs_kb, uint16_t* __restrict__ C, int64_t ldc,
    int64_t M, int64_t N, int64_t K, int mt, int nt, int c_vec) {
    __shared__ u32x4 sB[2][kBN * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    int tm, tn;
    tile_of(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t mw = m0 + kWM * wm;
    const int64_t nw = n0 + kWN * wn;
    const int64_t Kb = (K + kGroup - 1) / kGroup;
    const int64_t Kfull = K / kGroup;  // K-blocks with all 128 columns in range

    Operands op;
    {
        const int64_t arows = (M - m0) < kBM ? (M - m0) : kBM;
        const int64_t brows = (N - n0) < kBN ? (N - n0) : kBN;
        op.a = make_rsrc(A + m0 * lda, static_cast<uint32_t>(arows * lda));
        op.b = make_rsrc(B + n0 * ldb, static_cast<uint32_t>(brows * ldb));
        op.as = make_rsrc(a_s, static_cast<uint32_t>(M * Kb * 4));
        op.bs = make_rsrc(b_s, PER_COL ? static_cast<uint32_t>(N * Kb * 4) : 0u);
        op.a_lane = static_cast<uint32_t>((kWM * wm + l16) * lda + 32 * lg);
        op.b_lane = static_cast<uint32_t>((tid >> 3) * ldb + 16 * (tid & 7));
        op.a_sub = static_cast<uint32_t>(16 * lda);
        op.b_half = static_cast<uint32_t>(64 * ldb);
        op.b_eighth = static_cast<uint32_t>(8 * ldb);
        op.b_dma_lane = static_cast<uint32_t>((16 * wave + (lane >> 3)) * ldb + 16 * ((lane & 7) ^ (lane >> 3)));
#pragma unroll
        for (int i = 0; i < kMSub; ++i) {
            const int64_t m = mw + 16 * i + l16;
            op.as_off[i] = m < M ? static_cast<uint32_t>(4 * m) : kOob;
        }
        op.bs_partial = 0u;
#pragma unroll
        for (int j = 0; j < kNSub; ++j) {
            const int64_t n = nw + 16 * j + 4 * lg;
            op.bs_off[j] = n < N ? static_cast<uint32_t>(4 * n) : kOob;
            if (n < N && n + 4 > N) op.bs_partial |= 1u << j;
        }
    }

    v4f acc[kMSub][kNSub];
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
#pragma unroll
        for (int j = 0; j < kNSub; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (Kb > 0) {
        v8i af[2][kMSub];
        float as[2][kMSub];
        u32x4 bsv[2][kNSub];
        float bscal[2];

        // prologue: B(0) -> LDS[0]; A(0) and scales(0) -> registers
        if (Kfull > 0) {
            dma_b(sB[0], op, 0, wave);
            load_a<true>(af[0], op, 0, K, lg);
        } else {
            u32x4 bst[2];
            load_b<false>(bst, op, 0, K, tid);
            store_b(sB[0], bst, tid);
            load_a<false>(af[0], op, 0, K, lg);
        }
        load_scales<PER_COL>(as[0], bsv[0], bscal[0], op, b_s, bs_nb, bs_kb, 0, M, N, tn);
        __syncthreads();

        // One K-block; the buffer index is a compile-time constant so every register array stays
        // in registers. B(kb+1) streams into the other LDS buffer and A(kb+1) into the other
        // register set while this block computes; the barrier at the end publishes B(kb+1).
        auto step = [&](auto cur_tag, int64_t kb) {
            constexpr int cur = decltype(cur_tag)::value;
            constexpr int nxt = cur ^ 1;
            const bool more = kb + 1 < Kb;
            const bool next_full = kb + 1 < Kfull;
            auto issue_next = [&]() {
                if (more) {
                    if (next_full) {
                        dma_b(sB[nxt], op, kb + 1, wave);
                        load_a<true>(af[nxt], op, kb + 1, K, lg);
                    } else {
                        load_a<false>(af[nxt], op, kb + 1, K, lg);
                    }
                    load_scales<PER_COL>(as[nxt], bsv[nxt], bscal[nxt], op, b_s, bs_nb, bs_kb, kb + 1, M, N, tn);
                }
            };
            // fnuz: the next block's loads are issued once this block's A codes are all widened
            // (half way through, see below), so the two never hold registers together
            constexpr int kHalf = kMSub / 2;
            h8v ac[FNUZ ? kHalf : 1][4];
            if constexpr (!FNUZ) issue_next();
            // this K-block: partial products of every 16x16 subtile, rescaled into the totals.
            // Software pipeline over the 8 column subtiles: the B fragment of subtile j+1 is read
            // from LDS while subtile j's four MFMAs run, and subtile j-1's partials are rescaled
            // into the totals between them (one MFMA, then four FMAs).
            const u32x4* sb = sB[cur];
            float f[kMSub];
#pragma unroll
            for (int i = 0; i < kMSub; ++i) {
                f[i] = PER_COL ? as[cur][i] : as[cur][i] * bscal[cur];
                if (FNUZ) f[i] *= 16384.0f;  // 2^14: both widened operands carry 2^-7
            }
            auto read_bf = [&](int j) {
                const int r = kWN * wn + 16 * j + l16;
                return to_v8i(sb[r * 8 + ((2 * lg) ^ (r & 7))], sb[r * 8 + ((2 * lg + 1) ^ (r & 7))]);
            };
            auto rescale = [&](int j, const v4f (&pj)[kMSub]) {
#pragma unroll
                for (int i = 0; i < kMSub; ++i) {
                    if (PER_COL) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][e] = fmaf(pj[i][e], f[i] * __uint_as_float(bsv[cur][j][e]), acc[i][j][e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(pj[i][e], f[i], acc[i][j][e]);
                    }
                }
            };
            if constexpr (FNUZ) {
                // A widened to f16 takes twice the registers of its codes, so the wave's 64 rows are
                // done as two halves of 32: per half, the two A fragments are widened once and each
                // B fragment is read and widened once; one B fragment and one set of partials are
                // live at a time (the other wave of the SIMD covers the latencies).
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (h == 1) {
                        // the B fragments are read again rather than kept widened from the first
                        // half (the clobbers keep the compiler from merging the two reads), and the
                        // second half's A fragments pass through an empty asm here so that their
                        // widening cannot be hoisted into the first half
                        asm volatile("" ::: "memory");
#pragma unroll
                        for (int i = kHalf; i < kMSub; ++i)
#pragma unroll
                            for (int d = 0; d < 8; ++d) asm volatile("" : "+v"(af[cur][i][d]));
                    }
#pragma unroll
                    for (int i = 0; i < kHalf; ++i) fnuz_frag_to_f16(af[cur][h * kHalf + i], ac[i]);
                    if (h == 1) issue_next();
#pragma unroll
                    for (int j = 0; j < kNSub; ++j) {
                        // one B fragment in flight at a time (a memory clobber stops the compiler
                        // from hoisting the next fragment's read above this one's use)
                        if (j > 0) asm volatile("" ::: "memory");
                        h8v bc[4];
                        fnuz_frag_to_f16(read_bf(j), bc);
#pragma unroll
                        for (int i = 0; i < kHalf; ++i) {
                            const v4f p = mfma_f16_kblock(bc, ac[i]);
                            const int ii = h * kHalf + i;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float fe = PER_COL ? f[ii] * __uint_as_float(bsv[cur][j][e]) : f[ii];
                                acc[ii][j][e] = fmaf(p[e], fe, acc[ii][j][e]);
                            }
                        }
                    }
                }
            } else {
                v8i bf[2];
                v4f pp[2][kMSub];
                bf[0] = read_bf(0);
#pragma unroll
                for (int j = 0; j < kNSub; ++j) {
                    if (j + 1 < kNSub) bf[(j + 1) & 1] = read_bf(j + 1);
#pragma unroll
                    for (int i = 0; i < kMSub; ++i) pp[j & 1][i] = mfma_fp8_16x16x128(bf[j & 1], af[cur][i]);
                    if (j > 0) rescale(j - 1, pp[(j - 1) & 1]);
                }
                rescale(kNSub - 1, pp[(kNSub - 1) & 1]);
            }
            if (more && !next_full) {  // ragged last K-block: masked register path
                u32x4 bst[2];
                load_b<false>(bst, op, kb + 1, K, tid);
                store_b(sB[nxt], bst, tid);
            }
            __syncthreads();
        };
        for (int64_t kb = 0; kb < Kb; kb += 2) {
            step(IntTag<0>{}, kb);
            if (kb + 1 < Kb) step(IntTag<1>{}, kb + 1);
        }
    }

    // epilogue: lane holds C[m][n .. n+3] of every subtile
#pragma unroll
    for (int i = 0; i < kMSub; ++i) {
        const int64_t m = mw + 16 * i + l16;
        if (m >= M) continue;
        uint16_t* crow = C + m * ldc;
#pragma unroll
        for (int j = 0; j < kNSub; ++j) {
            const int64_t n = nw + 16 * j + 4 * lg;
            const uint32_t w0 = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t w1 = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            if (c_vec && n + 4 <= N) {
                *reinterpret_cast<uint2*>(crow + n) = make_uint2(w0, w1);
            } else {
                const uint16_t h[4] = {static_cast<uint16_t>(w0 & 0xFFFF), static_cast<uint16_t>(w0 >> 16),
                                       static_cast<uint16_t>(w1 & 0xFFFF), static_cast<uint16_t>(w1 >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) crow[n + e] = h[e];
            }
        }
    }
}

// ==============================================================================================
// Fast path (per-column scales: N % 4 == 0; 128x128 scales: at most 512 K-blocks): a 256 x 256
// workgroup tile of 8 waves, two per SIMD, each wave owning a 64 x 128 block of the tile (128 fp32
// totals in VGPRs).
//   * Every K-block's A tile (256 x 128 bytes), B tile (256 x 128 bytes) and scale slices go
//     global -> LDS by direct buffer loads (no registers) into one of two LDS stages, one K-block
//     ahead of the block being multiplied. Each wave loads 1/8 of every tile; the workgroup barrier
//     that follows each wave's wait for its own loads makes the stage visible to all.
//   * Two waves per SIMD: while one waits at the barrier or for LDS data, the other keeps the
//     matrix core busy. Per K-block and CU: 64 KB written to LDS and 192 KB read from it against
//     2048 MFMA cycles per SIMD.
//   * LDS rows hold their 16-byte chunks XOR-swizzled by (row / 2) % 8, so the 16 rows one fragment
//     read touches (per lane group) fall in 16 distinct groups of 4 banks.
namespace fast {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kWM = 64;
constexpr int kWN = 128;
constexpr int kWaves = 8;              // 4 (M) x 2 (N): two per SIMD
constexpr int kThreads = 64 * kWaves;  // 512
constexpr int kMSub = kWM / 16;        // 4
constexpr int kNSub = kWN / 16;        // 8
constexpr int kStages = 2;
constexpr int kMaxKbFast = 512;        // 128x128 B scales of the tile's columns, kept in LDS

// LDS image of one stage (16-byte units): A tile rows 0..255, B tile rows 0..255, then the A scales
// of the tile rows and the per-column B scales of the tile columns.
constexpr int kStageA = 0;
constexpr int kStageB = kStageA + kBM * 8;
constexpr int kStageSA = kStageB + kBN * 8;
constexpr int kStageSB = kStageSA + kBM / 4;
constexpr int kStageSize = kStageSB + kBN / 4;  // 4224 x 16 B = 66 KB

// vector-memory instructions each wave issues per stage: 4 A loads, 4 B loads (8 rows of 128 bytes
// each), the A scales and (per-column) the B scales of 32 rows / columns
constexpr int kLoadsPerStage(bool per_col) { return 4 + 4 + 1 + (per_col ? 1 : 0); }

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Expert grouping of one launch (MoE): kGroupRows -- experts own row ranges of A and C and bring
// their own B (forward, dgrad); kGroupK -- experts own token (K) ranges and write their own C
// (weight gradient).
constexpr int kGroupNone = 0;
constexpr int kGroupRows = 1;
constexpr int kGroupK = 2;
struct Grouping {
    const int64_t* offsets;  // E + 1 boundaries (device memory)
    int64_t E;
    int64_t b_stride;   // bytes between consecutive experts' B            (kGroupRows)
    int64_t bs_stride;  // floats between consecutive experts' B scales    (kGroupRows)
    int64_t c_stride;   // elements between consecutive experts' C         (kGroupK)
};

struct Ops {
    __amdgpu_buffer_rsrc_t a, b, as, bs;
    uint32_t a_lane[2];  // tile row 32 wave + lane / 8, chunk (lane % 8) ^ swz(row) for loads q even / odd
    uint32_t b_lane[2];  // same for B
    uint32_t as_lane;    // 4 (m0 + 32 wave + 4 lane): 4 A scales per lane (lanes 0..7)
    uint32_t bs_lane;    // 4 (n0 + 32 wave + 4 lane): 4 B scales per lane (lanes 0..7)
    uint32_t a_eighth;   // 8 lda
    uint32_t b_eighth;   // 8 ldb
    uint32_t lds;        // LDS byte address of stage 0
};

// One direct load, 16 bytes per lane to LDS address lds + 16 * lane; M0 is saved and restored.
__device__ __forceinline__ void dma16(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// The same for lanes 0 .. 7 only. A direct load writes LDS for every active lane (lanes whose offset
// is out of range write zeros), so the lanes beyond a scale slice are switched off; EXEC is changed
// and restored inside the asm block rather than through a branch, which would split the K-block's
// straight-line code.
__device__ __forceinline__ void dma16_8lanes(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    uint32_t saved_m0;
    uint64_t saved_exec;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_mov_b32 exec_lo, 0xff\n\t"
        "s_mov_b32 exec_hi, 0\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "buffer_load_dwordx4 %3, %4, %5 offen lds\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_mov_b64 exec, %1"
        : "=&s"(saved_m0), "=&s"(saved_exec)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory");
}

// Load number q of a stage, q = 0 .. kLoadsPerStage - 1: 0..3 A rows 32 wave + 8 q .., 4..7 B rows
// 32 wave + 8 (q - 4) .., 8 the A scales of rows 32 wave .. + 32, 9 (per-column) the B scales of
// columns 32 wave .. + 32. The loads of one stage can be spread over a K-block.
template <bool PER_COL>
__device__ __forceinline__ void issue_load(int q, const Ops& op, uint32_t stage_base, int64_t kb,
                                           int64_t M, int64_t N, int wave) {
    const uint32_t k = static_cast<uint32_t>(kb * kGroup);
    if (q < 4) {
        dma16(stage_base + (kStageA + (32 * wave + 8 * q) * 8) * 16, op.a, op.a_lane[q & 1], q * op.a_eighth + k);
    } else if (q < 8) {
        dma16(stage_base + (kStageB + (32 * wave + 8 * (q - 4)) * 8) * 16, op.b, op.b_lane[q & 1], (q - 4) * op.b_eighth + k);
    } else if (q == 8) {
        dma16_8lanes(stage_base + (kStageSA + 8 * wave) * 16, op.as, op.as_lane, static_cast<uint32_t>(kb * M * 4));
    } else if (PER_COL && q == 9) {
        dma16_8lanes(stage_base + (kStageSB + 8 * wave) * 16, op.bs, op.bs_lane, static_cast<uint32_t>(kb * N * 4));
    }
}

// Wait until at most N vector-memory instructions of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_own_loads() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// All LDS reads of this wave have returned, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool PER_COL, int GROUP>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ b_s, int64_t bs_nb,
    int64_t bs_kb, uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K, int mt,
    int nt, int c_vec, Grouping grp) {
    __shared__ u32x4 smem[kStages * kStageSize];
    __shared__ float bscale_lds[2][kMaxKbFast];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3;   // rows 64 wm .. of the tile
    const int wn = wave >> 2;  // columns 128 wn .. of the tile
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    int tm, tn;
    tile_of(blockIdx.x, mt, nt, tm, tn);
    int64_t m0 = static_cast<int64_t>(tm) * kBM;  // this tile's rows are [m0, min(m0 + kBM, m_end))
    int64_t m_end = M;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    // K-blocks (the last one may be partial: only for the ungrouped GEMMs, whose callers allow it)
    int64_t Kb = (K + kGroup - 1) / kGroup;
    if (GROUP == kGroupRows) {
        // tm indexes the concatenated row tiles of the experts; expert e owns rows
        // [offsets[e], offsets[e + 1]) of A and C (clamped to [0, M] and made non-decreasing) and
        // multiplies them by its own B and B scales
        int64_t first = 0, lo = 0, hi = 0;
        int64_t e = -1;
        int64_t prev = 0;
        for (int64_t j = 0; j < grp.E; ++j) {
            const int64_t a = min(max(grp.offsets[j], prev), M);
            const int64_t b = min(max(grp.offsets[j + 1], a), M);
            prev = b;
            const int64_t tiles = (b - a + kBM - 1) / kBM;
            if (tm < first + tiles) {
                e = j;
                lo = a;
                hi = b;
                break;
            }
            first += tiles;
        }
        if (e < 0) return;  // a spare workgroup of the grid's upper bound: the whole group leaves
        m0 = lo + (tm - first) * kBM;
        m_end = hi;
        B += e * grp.b_stride;
        b_s += e * grp.bs_stride;
    } else if (GROUP == kGroupK) {
        // expert e = blockIdx.y owns the K-blocks [offsets[e] / 128, offsets[e + 1] / 128) of A and B
        // (token ranges of the weight gradient) and writes its own C
        const int64_t e = blockIdx.y;
        const int64_t lo = min(max(grp.offsets[e], int64_t{0}), K);
        const int64_t hi = min(max(grp.offsets[e + 1], lo), K);
        const int64_t kb0 = lo / kGroup;
        Kb = hi / kGroup - kb0;
        A += kb0 * kGroup;
        B += kb0 * kGroup;
        a_s += kb0 * M;
        b_s += PER_COL ? kb0 * N : kb0 * bs_kb;
        C += e * grp.c_stride;
    }
    constexpr int kLoads = kLoadsPerStage(PER_COL);

    Ops op;
    {
        const int64_t arows = (m_end - m0) < kBM ? (m_end - m0) : kBM;
        const int64_t brows = (N - n0) < kBN ? (N - n0) : kBN;
        op.a = make_rsrc(A + m0 * lda, static_cast<uint32_t>(arows * lda));
        op.b = make_rsrc(B + n0 * ldb, static_cast<uint32_t>(brows * ldb));
        op.as = make_rsrc(a_s, static_cast<uint32_t>(M * Kb * 4));
        op.bs = make_rsrc(b_s, PER_COL ? static_cast<uint32_t>(N * Kb * 4) : 0u);
        // row 32 wave + 8 q + lane / 8 has swz = (4 q + lane / 16) % 8, which depends on q % 2
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int chunk = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
            op.a_lane[par] = static_cast<uint32_t>((32 * wave + (lane >> 3)) * lda + 16 * chunk);
            op.b_lane[par] = static_cast<uint32_t>((32 * wave + (lane >> 3)) * ldb + 16 * chunk);
        }
        op.as_lane = static_cast<uint32_t>(4 * (m0 + 32 * wave + 4 * lane));
        op.bs_lane = static_cast<uint32_t>(4 * (n0 + 32 * wave + 4 * lane));
        op.a_eighth = static_cast<uint32_t>(8 * lda);
        op.b_eighth = static_cast<uint32_t>(8 * ldb);
        op.lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)));
    }

    v4f acc[kMSub][kNSub];
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
#pragma unroll
        for (int j = 0; j < kNSub; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (Kb > 0) {
        auto stage_base = [&](int stage) { return op.lds + static_cast<uint32_t>(stage * kStageSize * 16); };
        // Fragment lane (l16, lg) holds 16-byte chunks lg and lg + 4 of its row (row bytes
        // [16 lg, 16 lg + 16) and [64 + 16 lg, 64 + 16 lg + 16)). Any assignment of a row's 128
        // bytes to the four lane groups' 32 operand bytes gives the same dot product as long as A
        // and B use the same one; this one makes every ds_read_b128 conflict free at the full LDS
        // rate (4 cycles per instruction on gfx950, where chunks 2 lg and 2 lg + 1 take 8).
        const int sw = swz(l16);  // the same for every fragment row 16 x + l16
        const int pos_lo = lg ^ sw;
        const int pos_hi = (lg + 4) ^ sw;

        // prologue: block 0 into stage 0
#pragma unroll
        for (int q = 0; q < kLoads; ++q) issue_load<PER_COL>(q, op, stage_base(0), 0, M, N, wave);

        // 128x128 B scales of the tile's two 128-column blocks for every K-block, fetched while
        // block 0 is in flight (their wait covers both)
        if (!PER_COL) {
            for (int64_t c = tid; c < 2 * Kb; c += kThreads) {
                const int half = c >= Kb;
                const int64_t kb = c - half * Kb;
                const int64_t nb = 2 * static_cast<int64_t>(tn) + half;
                // a column block past N is never stored; read block 0's scale instead
                bscale_lds[half][kb] = b_s[(nb * kGroup < N ? nb : 0) * bs_nb + kb * bs_kb];
            }
        }
        wait_own_loads<0>();

        // Bytes of the last K-block that lie below K (128 when K % 128 == 0). Its DMA loads read whole
        // 128-byte rows, so bytes at and past K (row padding, or the start of the next row) are
        // zeroed in the fragment registers of that block: register d of lane group lg holds row
        // bytes from 16 lg + 4 d (d < 4) and from 64 + 16 lg + 4 (d - 4) (d >= 4), in both operands.
        const int krem = static_cast<int>(K - (Kb - 1) * kGroup);
        const int lane_keep = krem - 16 * lg;
        auto tail_mask = [&](v8i v) {
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int keep = lane_keep - (d < 4 ? 4 * d : 64 + 4 * (d - 4));
                const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
                v[d] = static_cast<int>(static_cast<uint32_t>(v[d]) & m);
            }
            return v;
        };

        // One loop body for both stages (stage = kb % 2 at run time): a body unrolled per stage
        // makes the register allocator spill. TAIL: the partial last K-block (fragments masked).
        auto step = [&](int64_t kb, auto tail_tag) {
            constexpr bool TAIL = decltype(tail_tag)::value;
            const int cur = static_cast<int>(kb & 1);
            const int nxt = cur ^ 1;
            // every wave's block-kb loads are in LDS, and every wave is done with block kb-1
            lds_barrier();
            const uint32_t base_n = stage_base(nxt);
            const int64_t kb_next = kb + 1 < Kb ? kb + 1 : kb;  // past the end: reload (unused)

            const u32x4* st = smem + cur * kStageSize;
            const float* sa = reinterpret_cast<const float*>(st + kStageSA) + 64 * wm;
            const float* sbs = reinterpret_cast<const float*>(st + kStageSB) + 128 * wn;
            auto read_bf = [&](int j) {
                const int r = 128 * wn + 16 * j + l16;
                const v8i v = to_v8i(st[kStageB + r * 8 + pos_lo], st[kStageB + r * 8 + pos_hi]);
                return TAIL ? tail_mask(v) : v;
            };
            // B fragments are read two subtiles ahead of their MFMAs (three in registers); the
            // first MFMA needs only bf[0] and af[0], so those are read first
            v8i bf[3];
            v8i af[kMSub];
            bf[0] = read_bf(0);
#pragma unroll
            for (int i = 0; i < kMSub; ++i) {
                const int r = 64 * wm + 16 * i + l16;
                af[i] = to_v8i(st[kStageA + r * 8 + pos_lo], st[kStageA + r * 8 + pos_hi]);
                if (TAIL) af[i] = tail_mask(af[i]);
            }
            bf[1] = read_bf(1);
            const float bsc = PER_COL ? 1.0f : bscale_lds[wn][kb];
            float f[kMSub];
#pragma unroll
            for (int i = 0; i < kMSub; ++i) f[i] = PER_COL ? sa[16 * i + l16] : sa[16 * i + l16] * bsc;

            // partial of subtile (i, j) times its scales, into the totals
            auto rescale = [&](int i, int j, const v4f& p, const v4f& bsj) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] = fmaf(p[e], PER_COL ? f[i] * bsj[e] : f[i], acc[i][j][e]);
            };
            auto read_bsj = [&](int j) {
                return PER_COL ? *reinterpret_cast<const v4f*>(sbs + 16 * j + 4 * lg) : v4f{1.0f, 1.0f, 1.0f, 1.0f};
            };
            v4f pp[kMSub];  // partials of the previous subtile until rescaled, then of the current one
            v4f bsj_prev = {1.0f, 1.0f, 1.0f, 1.0f};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kNSub; ++j) {
                // the next block's loads, spread over the first subtiles
                if (2 * j < kLoads) issue_load<PER_COL>(2 * j, op, base_n, kb_next, M, N, wave);
                if (2 * j + 1 < kLoads) issue_load<PER_COL>(2 * j + 1, op, base_n, kb_next, M, N, wave);
                if (j + 2 < kNSub) bf[(j + 2) % 3] = read_bf(j + 2);
                const v4f bsj = read_bsj(j);
                // the previous subtile's partial of row block i is rescaled just before the MFMA
                // that overwrites it (4 MFMAs after the one that produced it)
#pragma unroll
                for (int i = 0; i < kMSub; ++i) {
                    if (j > 0) rescale(i, j - 1, pp[i], bsj_prev);
                    pp[i] = mfma_fp8_16x16x128(bf[j % 3], af[i]);
                }
                bsj_prev = bsj;
                if (j + 2 < kNSub) __builtin_amdgcn_sched_group_barrier(0x100, PER_COL ? 3 : 2, 0);
#pragma unroll
                for (int i = 0; i < kMSub; ++i) {
                    if (j > 0) __builtin_amdgcn_sched_group_barrier(0x002, PER_COL ? 8 : 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < kMSub; ++i) rescale(i, kNSub - 1, pp[i], bsj_prev);
            wait_own_loads<0>();  // this wave's loads of block kb+1 have landed
        };

        const int64_t Kb_full = krem == kGroup ? Kb : Kb - 1;
        for (int64_t kb = 0; kb < Kb_full; ++kb) step(kb, std::false_type{});
        if (Kb_full < Kb) step(Kb_full, std::true_type{});
    }

    // Epilogue: each wave's 64 x 128 bf16 block goes through LDS (the stages are free once every
    // wave has left the K-loop), so the global stores are 16 bytes per lane and whole 128-byte
    // lines (a lane's own outputs are 4 columns of one row). Row r of a block holds 16 chunks of 16
    // bytes, chunk c at position c ^ (r % 16), which keeps both LDS passes free of bank conflicts.
    __syncthreads();
    uint8_t* cblk = reinterpret_cast<uint8_t*>(smem) + wave * (kWM * kWN * 2);
#pragma unroll
    for (int i = 0; i < kMSub; ++i) {
        const int r = 16 * i + l16;
#pragma unroll
        for (int j = 0; j < kNSub; ++j) {
            const uint32_t w0 = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t w1 = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            const int chunk = 2 * j + (lg >> 1);
            *reinterpret_cast<uint2*>(cblk + r * 256 + ((chunk ^ (r & 15)) * 16) + 8 * (lg & 1)) =
                make_uint2(w0, w1);
        }
    }
    const int cc = lane & 15;  // 16-byte chunk (8 columns) of a row
#pragma unroll
    for (int p = 0; p < kWM / 4; ++p) {
        const int r = 4 * p + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(cblk + r * 256 + ((cc ^ (r & 15)) * 16));
        const int64_t m = m0 + 64 * wm + r;
        if (m >= m_end) continue;
        const int64_t n = n0 + 128 * wn + 8 * cc;
        uint16_t* dst = C + m * ldc + n;
        if (c_vec && n + 8 <= N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace fast

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                       int64_t ldb, BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N,
                       int64_t K, bool fnuz, hipStream_t stream) {
    // vector stores: 8 bytes per lane in the general kernel, 16 in the fast one
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 8 == 0) && (ldc % 4 == 0);
    const int c_vec16 = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
    // Fast path: per-column scales read 4 columns at a time; 128x128 scales of a
    // tile's column staged in LDS (at most kMaxKbFast K-blocks).
    const bool fast_scales = bs.per_column ? (N % 4 == 0) : ((K + kGroup - 1) / kGroup <= fast::kMaxKbFast);
    if (!fnuz && fast_scales) {
        const int64_t mt = (M + fast::kBM - 1) / fast::kBM;
        const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
        if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(mt * nt));
        const fast::Grouping none{nullptr, 0, 0, 0, 0};
        if (bs.per_column)
            fast::gemm_kernel<true, fast::kGroupNone><<<grid, fast::kThreads, 0, stream>>>(
                a, lda, a_s, b, ldb, bs.ptr, 0, 0, c, ldc, M, N, K, (int)mt, (int)nt, c_vec16, none);
        else
            fast::gemm_kernel<false, fast::kGroupNone><<<grid, fast::kThreads, 0, stream>>>(
                a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb, bs.stride_kb, c, ldc, M, N, K, (int)mt,
                (int)nt, c_vec16, none);
        return hipGetLastError();
    }
    const int64_t mt = (M + kBM - 1) / kBM;
    const int64_t nt = (N + kBN - 1) / kBN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(mt * nt));
    const int64_t nb_stride = bs.per_column ? 0 : bs.stride_nb;
    const int64_t kb_stride = bs.per_column ? 0 : bs.stride_kb;
#define BSFP8_GG(PC, FZ)                                                                          \
    gemm_kernel<PC, FZ><<<grid, kThreads, 0, stream>>>(a, lda, a_s, b, ldb, bs.ptr, nb_stride,    \
                                                       kb_stride, c, ldc, M, N, K, (int)mt,       \
                                                       (int)nt, c_vec)
    if (bs.per_column) {
        if (fnuz) BSFP8_GG(true, true);
        else BSFP8_GG(true, false);
    } else {
        if (fnuz) BSFP8_GG(false, true);
        else BSFP8_GG(false, false);
    }
#undef BSFP8_GG
    return hipGetLastError();
}

bool gemm_grouped_supported(bool per_column, int64_t N, int64_t K) {
    if (K % kGroup != 0) return false;
    return per_column ? (N % 4 == 0) : (K / kGroup <= fast::kMaxKbFast);
}

hipError_t launch_gemm_grouped_rows(const uint8_t* a, int64_t lda, const float* a_s,
                                    const uint8_t* b, int64_t ldb, int64_t b_stride, BScale bs,
                                    int64_t bs_stride, const int64_t* offsets, int64_t E,
                                    uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                    hipStream_t stream) {
    if (!gemm_grouped_supported(false, N, K)) return hipErrorInvalidValue;
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
    // every expert's last row tile may be partial: at most ceil(M / 256) + E row tiles
    const int64_t mt = (M + fast::kBM - 1) / fast::kBM + E;
    const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const fast::Grouping g{offsets, E, b_stride, bs_stride, 0};
    fast::gemm_kernel<false, fast::kGroupRows><<<dim3(static_cast<unsigned>(mt * nt)), fast::kThreads, 0, stream>>>(
        a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb, bs.stride_kb, c, ldc, M, N, K, (int)mt, (int)nt,
        c_vec, g);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped_k(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                                 int64_t ldb, const float* b_s, const int64_t* offsets, int64_t E,
                                 uint16_t* c, int64_t ldc, int64_t c_stride, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream) {
    if (!gemm_grouped_supported(true, N, K)) return hipErrorInvalidValue;
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0) && (c_stride % 8 == 0);
    const int64_t mt = (M + fast::kBM - 1) / fast::kBM;
    const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
    if (mt * nt > 0x7FFFFFFFLL || E > 65535) return hipErrorInvalidValue;
    const fast::Grouping g{offsets, E, 0, 0, c_stride};
    fast::gemm_kernel<true, fast::kGroupK><<<dim3(static_cast<unsigned>(mt * nt), static_cast<unsigned>(E)), fast::kThreads, 0, stream>>>(
        a, lda, a_s, b, ldb, b_s, 0, 0, c, ldc, M, N, K, (int)mt, (int)nt, c_vec, g);
    return hipGetLastError();
}

}  // namespace bsfp8
