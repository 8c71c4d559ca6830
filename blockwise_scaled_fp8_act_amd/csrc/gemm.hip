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
//     of one row m: the 128x128 rescale factor is one scalar per (lane, 16-row subtile) and a lane
//     holds 8 contiguous bytes of a bf16 output row;
//   * every operand and scale is read through a raw buffer resource with the whole offset in the
//     per-lane register, and a lane whose row, column or scale lies outside the tensor gets an
//     out-of-range offset (geometry.hpp, whose arithmetic the CPU tests enumerate lane by lane);
//     outputs of rows >= M or columns >= N are never stored.
// The fast kernel (namespace fast) serves the float8_e4m3fn GEMMs, a partial last K-block
// included, in 256 x 256 tiles, or in 128 x 256 tiles when the larger ones would leave CUs idle;
// the thin kernel (namespace thin) serves short-and-wide shapes whose 128-row tiles would fill at
// most half the CUs, in 64-row tiles over the whole K range; when even those are few and K is long,
// the fast kernel splits K over several workgroups per tile (fp32 partial tiles, summed by a second
// kernel). The rules are in schedule.hpp. The general kernel (namespace gen) serves the
// float8_e4m3fnuz operands. All zero the bytes of a partial last K-block that lie at or past K.
//
// float8_e4m3fnuz operands (the format of the ROCm page's MI300X runs, FP8_MAX 240): gfx950's FP8
// matrix instructions read e4m3fn, and no power-of-two rescaling maps every fnuz value onto an
// e4m3fn value (fnuz spans 2^-10 .. 240, e4m3fn 2^-9 .. 448, and 2 x 240 = 480 is not an e4m3fn
// value). Each fnuz code is instead widened exactly to f16 in registers (its 7 magnitude bits placed
// under the f16 exponent field: the value times 2^-7, the smallest ones as f16 subnormals) and a
// K-block is four v_mfma_f32_16x16x32_f16 instead of one FP8 instruction -- products of two
// 4-significant-bit values are exact in fp32 either way, so the per-K-block partials equal the fn
// path's arithmetic up to the exact factor 2^-14.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace bsfp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef short s2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
        const u32x4 h = {fnuz2_to_f16x2<0>(w0), fnuz2_to_f16x2<1>(w0), fnuz2_to_f16x2<0>(w1), fnuz2_to_f16x2<1>(w1)};
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

// Raw buffer resource over [base, base + bytes): loads at per-lane offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, static_cast<int>(bytes),
                                             0x00020000);
}

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

typedef __attribute__((address_space(3))) void lds_void_t;

// ==============================================================================================
// General kernel (float8_e4m3fnuz operands): a 256 x 128 workgroup tile of 8 waves, each a 64 x 64
// block; A fragments and scales are loaded into registers, B tiles through LDS.
namespace gen {

constexpr int kBM = geom::kGenBM;
constexpr int kBN = geom::kGenBN;
constexpr int kWM = 64;
constexpr int kWN = 64;
constexpr int kThreads = 512;   // two waves per SIMD
constexpr int kMSub = kWM / 16;
constexpr int kNSub = kWN / 16;

// Per-workgroup addressing state (geometry.hpp): A subtile i, B register rows p and B direct-load q
// read through resources that start at their first tile row and end at the matrix edge; scale
// reads carry a per-lane base (kOob outside the tensor) plus a per-K-block advance.
struct Operands {
    __amdgpu_buffer_rsrc_t a[kMSub], b_reg[2], b_dma[2], as, bs;
    uint32_t a_lane, b_lane, bdma_lane;
    uint32_t as_base[kMSub];  // geom::gen_ascale_base
    uint32_t bs_col;          // geom::gen_bscale_tile_base (per-column scales, staged in LDS)
    int64_t M, N;
};

// A operand of K-block kb for this lane: subtile i covers rows 16 i + l16 of the wave's 64 rows and
// bytes [32 lg, 32 lg + 32) of the block, exactly the MFMA's per-lane operand layout.
template <bool FULL>
__device__ __forceinline__ void load_a(v8i (&af)[kMSub], const Operands& op, int64_t kb, int64_t K, int lane) {
    const int lg = lane >> 4;
    const uint32_t off = op.a_lane + static_cast<uint32_t>(kb * kGroup);
#pragma unroll
    for (int i = 0; i < kMSub; ++i) {
        u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(op.a[i], off, 0, 0);
        u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(op.a[i], off + 16, 0, 0);
        if (!FULL) {
            const int64_t valid = K - (kb * kGroup + 32 * lg);
            lo = mask_tail(lo, valid);
            hi = mask_tail(hi, valid - 16);
        }
        af[i] = to_v8i(lo, hi);
    }
}

// B tile of a partial K-block (128 rows x 128 bytes) into registers, bytes past K zeroed.
__device__ __forceinline__ void load_b_tail(u32x4 (&bst)[2], const Operands& op, int64_t kb, int64_t K, int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(op.b_reg[p], op.b_lane + static_cast<uint32_t>(kb * kGroup), 0, 0);
        bst[p] = mask_tail(v, K - (kb * kGroup + 16 * (tid & 7)));
    }
}

// LDS image of a B tile: row r, 16-byte chunk c stored at chunk position c ^ (r % 8), so the
// fragment reads (rows 16 j .. 16 j + 15 at one logical chunk) spread over all banks.
__device__ __forceinline__ void store_b(u32x4* __restrict__ sb, const u32x4 (&bst)[2], int tid) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = geom::gen_b_row(tid, p);
        const int ch = tid & 7;
        sb[r * 8 + (ch ^ (r & 7))] = bst[p];
    }
}

// B tile of a full K-block straight from global memory into its LDS image (no registers): wave w
// fills tile rows [16 w, 16 w + 16) with two 1 KB loads.
__device__ __forceinline__ void dma_b(u32x4* __restrict__ sb, const Operands& op, int64_t kb, int wave) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        lds_void_t* dst = (lds_void_t*)(sb + (16 * wave + 8 * q) * 8);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op.b_dma[q], dst, 16, op.bdma_lane + static_cast<uint32_t>(kb * kGroup), 0, 0, 0);
    }
}

// Scales of K-block kb: the lane's four A-row scales into registers; per column, the thread's one
// tile-column scale (threads 0..127; the others read nothing useful and store nothing), which the
// kernel stages in LDS; 128x128, the tile's one column-block scale.
template <bool PER_COL>
__device__ __forceinline__ void load_scales(float (&as)[kMSub], float& bcol, float& bscal,
                                            const Operands& op, const float* __restrict__ b_s,
                                            int64_t bs_nb, int64_t bs_kb, int64_t kb, int tn) {
    const uint32_t acol = static_cast<uint32_t>(4 * kb * op.M);
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
        as[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(op.as, op.as_base[i] + acol, 0, 0));
    if (PER_COL) {
        bcol = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(op.bs, op.bs_col + static_cast<uint32_t>(4 * kb * op.N), 0, 0));
    } else {
        // the tile's one 128-column block (tiles exist only for columns below N)
        bscal = b_s[static_cast<int64_t>(tn) * bs_nb + kb * bs_kb];
    }
}

template <bool PER_COL>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ b_s,
    int64_t bs_nb, int64_t bs_kb, uint16_t* __restrict__ C, int64_t ldc,
    int64_t M, int64_t N, int64_t K, int mt, int nt, int c_vec) {
    __shared__ u32x4 sB[2][kBN * 8];
    __shared__ float sBS[2][kBN];  // per-column B scales of the two K-blocks in flight

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    int tm, tn;
    geom::tile_of(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t Kb = (K + kGroup - 1) / kGroup;
    const int64_t Kfull = K / kGroup;  // K-blocks with all 128 columns in range

    Operands op;
    {
        const int64_t arows = (M - m0) < kBM ? (M - m0) : kBM;
        const int64_t brows = (N - n0) < kBN ? (N - n0) : kBN;
#pragma unroll
        for (int i = 0; i < kMSub; ++i)
            op.a[i] = make_rsrc(A + (m0 + geom::gen_a_first_row(i)) * lda, geom::gen_a_range(i, arows, lda));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            op.b_reg[p] = make_rsrc(B + (n0 + geom::gen_b_first_row(p)) * ldb, geom::gen_b_range(p, brows, ldb));
            op.b_dma[p] = make_rsrc(B + (n0 + geom::gen_bdma_first_row(p)) * ldb, geom::gen_bdma_range(p, brows, ldb));
        }
        op.as = make_rsrc(a_s, M * Kb * 4);
        op.bs = make_rsrc(b_s, PER_COL ? N * Kb * 4 : 0);
        op.a_lane = geom::gen_a_lane(wm, lane, lda);
        op.b_lane = geom::gen_b_lane(tid, ldb);
        op.bdma_lane = geom::gen_bdma_lane(wave, lane, ldb);
#pragma unroll
        for (int i = 0; i < kMSub; ++i) op.as_base[i] = geom::gen_ascale_base(m0, wm, i, lane, M);
        op.bs_col = geom::gen_bscale_tile_base(n0, N, tid);
        op.M = M;
        op.N = N;
    }

    v4f acc[kMSub][kNSub];
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
#pragma unroll
        for (int j = 0; j < kNSub; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (Kb > 0) {
        v8i af[2][kMSub];
        float as[2][kMSub];
        float bcol[2];
        float bscal[2];

        // prologue: B(0) -> LDS[0]; A(0) and scales(0) -> registers
        if (Kfull > 0) {
            dma_b(sB[0], op, 0, wave);
            load_a<true>(af[0], op, 0, K, lane);
        } else {
            u32x4 bst[2];
            load_b_tail(bst, op, 0, K, tid);
            store_b(sB[0], bst, tid);
            load_a<false>(af[0], op, 0, K, lane);
        }
        load_scales<PER_COL>(as[0], bcol[0], bscal[0], op, b_s, bs_nb, bs_kb, 0, tn);
        if (PER_COL && tid < kBN) sBS[0][tid] = bcol[0];
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
                        load_a<true>(af[nxt], op, kb + 1, K, lane);
                    } else {
                        load_a<false>(af[nxt], op, kb + 1, K, lane);
                    }
                    load_scales<PER_COL>(as[nxt], bcol[nxt], bscal[nxt], op, b_s, bs_nb, bs_kb, kb + 1, tn);
                }
            };
            // the next block's loads are issued once this block's A codes are all widened (half
            // way through, see below), so the two never hold registers together
            constexpr int kHalf = kMSub / 2;
            h8v ac[kHalf][4];
            const u32x4* sb = sB[cur];
            float f[kMSub];
#pragma unroll
            for (int i = 0; i < kMSub; ++i) {
                f[i] = PER_COL ? as[cur][i] : as[cur][i] * bscal[cur];
                f[i] *= 16384.0f;  // 2^14: both widened operands carry 2^-7
            }
            auto read_bf = [&](int j) {
                const int r = kWN * wn + 16 * j + l16;
                return to_v8i(sb[r * 8 + ((2 * lg) ^ (r & 7))], sb[r * 8 + ((2 * lg + 1) ^ (r & 7))]);
            };
            // A widened to f16 takes twice the registers of its codes, so the wave's 64 rows are
            // done as two halves of 32: per half, the two A fragments are widened once and each B
            // fragment is read and widened once; one B fragment and one set of partials are live
            // at a time (the other wave of the SIMD covers the latencies).
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1) {
                    // the B fragments are read again rather than kept widened from the first half
                    // (the clobbers keep the compiler from merging the two reads), and the second
                    // half's A fragments pass through an empty asm here so that their widening
                    // cannot be hoisted into the first half
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
                    // one B fragment in flight at a time (a memory clobber stops the compiler from
                    // hoisting the next fragment's read above this one's use)
                    if (j > 0) asm volatile("" ::: "memory");
                    h8v bc[4];
                    fnuz_frag_to_f16(read_bf(j), bc);
                    // per column: the scales of the lane's four columns of subtile j
                    const v4f bsj = PER_COL ? *reinterpret_cast<const v4f*>(&sBS[cur][kWN * wn + 16 * j + 4 * lg])
                                            : v4f{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
                    for (int i = 0; i < kHalf; ++i) {
                        const v4f p = mfma_f16_kblock(bc, ac[i]);
                        const int ii = h * kHalf + i;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float fe = PER_COL ? f[ii] * bsj[e] : f[ii];
                            acc[ii][j][e] = fmaf(p[e], fe, acc[ii][j][e]);
                        }
                    }
                }
            }
            if (more && !next_full) {  // ragged last K-block: masked register path
                u32x4 bst[2];
                load_b_tail(bst, op, kb + 1, K, tid);
                store_b(sB[nxt], bst, tid);
            }
            // the next block's per-column scales (sBS[nxt] was last read in the previous step)
            if (PER_COL && more && tid < kBN) sBS[nxt][tid] = bcol[nxt];
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
        const int64_t m = m0 + geom::gen_a_row(wm, i, lane);
        if (m >= M) continue;
        uint16_t* crow = C + m * ldc;
#pragma unroll
        for (int j = 0; j < kNSub; ++j) {
            const int64_t n = geom::gen_col(n0, wn, j, lane);
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

}  // namespace gen

// ==============================================================================================
// Fast kernel: a 256 x 256 workgroup tile of 8 waves, two per SIMD, each wave owning a 64 x 128
// block of the tile (128 fp32 totals in VGPRs); the 128 x 256 tile has 8 waves of 32 x 128. The
// figures below are those of the 256-row tile.
//   * Every K-block's A tile (256 x 128 bytes), B tile (256 x 128 bytes) and scale slices go
//     global -> LDS by direct buffer loads (no registers) into one of two LDS stages. Each wave
//     loads 1/8 of every tile; a workgroup barrier that follows each wave's wait for its own loads
//     makes a stage visible to all.
//   * Two waves per SIMD: while one waits at the barrier or for LDS data, the other keeps the
//     matrix core busy. Per K-block and CU: 64 KB written to LDS and 192 KB read from it against
//     2048 MFMA cycles per SIMD.
//   * LDS rows hold their 16-byte chunks XOR-swizzled by (row / 2) % 8, so the 16 rows one fragment
//     read touches (per lane group) fall in 16 distinct groups of 4 banks.
namespace fast {

constexpr int kBN = geom::kFastBN;
constexpr int kWM = 64;                   // wave block rows of the 256-row tile
constexpr int kWMSmall = 32;              // ... of the 128-row tile (8 waves, two per SIMD)
constexpr int kWN = 128;
constexpr int kNSub = kWN / 16;           // 8
constexpr int kStages = 2;

// Tile geometry for tile height BM and wave block height WM (each wave computes a WM x 128 block):
// BM 256, WM 64 -- 8 waves, 4 (M) x 2 (N), two per SIMD; BM 128, WM 32 -- 8 waves, 4 x 2, two per
// SIMD, for problems whose 256-row tiles would leave compute units idle (10-17% faster than 4 waves
// of 64 x 128, one per SIMD, which the template also describes: 2048 x 4096 x 4096 37.3 against
// 43.0 us).
template <int BM, int WM = kWM>
struct Cfg {
    static constexpr int kWaveM = WM;
    static constexpr int kMSub = WM / 16;       // 16-row subtiles per wave
    static constexpr int kWavesM = BM / WM;
    static constexpr int kWaves = 2 * kWavesM;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kARows = BM / kWaves;  // A rows (and A scales) a wave loads: 32 or 16
    static constexpr int kALoads = kARows / 8;
    static constexpr int kBRows = kBN / kWaves;  // B rows (and per-column B scales) a wave loads: 32 or 64
    static constexpr int kBLoads = kBRows / 8;
    // LDS image of one stage (16-byte units): A tile rows 0..BM-1, B tile rows 0..255, then the A
    // scales of the tile rows and the B scales (per column: of the tile columns; 128x128: of the
    // tile's two column blocks, floats 0 and 1). BM 256: 4224 units (66 KB); BM 128: 3168 (49.5 KB).
    static constexpr int kStageA = 0;
    static constexpr int kStageB = kStageA + BM * 8;
    static constexpr int kStageSA = kStageB + kBN * 8;
    static constexpr int kStageSB = kStageSA + BM / 4;
    static constexpr int kStageSize = kStageSB + kBN / 4;
    // vector-memory instructions each wave issues per stage: kALoads A loads and kBLoads B loads (8
    // rows of 128 bytes each), the A scales of kARows rows, the B scales (kBRows columns, or the two
    // column-block scales)
    static constexpr int kLoads = kALoads + kBLoads + 2;
    // a block's loads past the first four are issued two per subtile column over this many columns
    static constexpr int kPendCols = (kLoads - 3) / 2;
};
constexpr int kBM = geom::kFastBM;
constexpr int kBMSmall = geom::kFastBMSmall;

// One launch's work split: kGroupRows -- experts own row ranges of A and C and bring their own B
// (forward, dgrad); kGroupK -- experts own token (K) ranges and write their own C (weight
// gradient); kSplitK -- slice blockIdx.y of gridDim.y owns a range of K-blocks and writes an fp32
// partial tile (summed by split_reduce_kernel).
constexpr int kGroupNone = 0;
constexpr int kGroupRows = 1;
constexpr int kGroupK = 2;
constexpr int kSplitK = 3;
struct Grouping {
    const int64_t* offsets;  // E + 1 boundaries (device memory)
    int64_t E;
    int64_t b_stride;   // bytes between consecutive experts' B            (kGroupRows)
    int64_t bs_stride;  // floats between consecutive experts' B scales    (kGroupRows)
    int64_t c_stride;   // elements between consecutive experts' C (kGroupK); floats per partial (kSplitK)
    int32_t* status;    // kGroupK: set to 1 when an expert's token range is not 128-aligned (may be null)
};

struct Ops {
    __amdgpu_buffer_rsrc_t a[4], b[4];  // operand load q reads through a[q % 4] / b[q % 4] (from tile row 8 (q % 4))
    __amdgpu_buffer_rsrc_t as, bs;
    uint32_t a_lane[2];  // geom::fast_operand_lane for loads with q % 2 = 0 / 1
    uint32_t b_lane[4];  // ... for B loads with q % 2 + 2 (q / 4) = 0 .. 3
    uint32_t as_base;    // geom::fast_ascale_base
    uint32_t bs_base;    // geom::fast_bscale_col_base / fast_bscale_blk_base
    int64_t as_step;     // bytes between K-blocks of the A scales (4 M)
    int64_t bs_step;     // ... of the B scales (4 N per column; 4 bs_kb for 128x128)
    uint32_t lds;        // LDS byte address of stage 0
};

// A wave-uniform 64-bit lane mask in scalar registers. readfirstlane returns a signed int: each half
// goes through uint32_t so a low half with bit 31 set does not sign-extend into the high half.
__device__ __forceinline__ uint64_t uniform_mask(uint64_t lanes) {
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(lanes >> 32)));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(lanes)));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One direct load to LDS address lds + 16 * lane (16 bytes per lane), for the lanes set in both
// EXEC and `lanes` (a wave-uniform mask); the scalar offset is zero. A direct load writes LDS for
// every active lane (lanes whose offset is out of range write zeros), so every lane of a load that
// is not wanted is switched off. EXEC and M0 are changed and restored inside the asm block rather
// than through a branch, which would split the K-block's straight-line code (a uniform branch there
// makes the register allocator spill).
__device__ __forceinline__ void dma16(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint64_t lanes) {
    uint32_t saved_m0;
    uint64_t saved_exec;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_and_b64 exec, exec, %5\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "buffer_load_dwordx4 %3, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_mov_b64 exec, %1"
        : "=&s"(saved_m0), "=&s"(saved_exec)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(uniform_mask(lanes))
        : "memory");
}

// The same with 4 bytes per lane, to LDS address lds + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint64_t lanes) {
    uint32_t saved_m0;
    uint64_t saved_exec;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_and_b64 exec, exec, %5\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "buffer_load_dword %3, %4, 0 offen lds\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_mov_b64 exec, %1"
        : "=&s"(saved_m0), "=&s"(saved_exec)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r), "s"(uniform_mask(lanes))
        : "memory");
}

// Load number q of a stage, q = 0 .. kLoads - 1: kALoads A loads of rows kARows wave + 8 q .., then
// kBLoads B loads of rows kBRows wave + 8 (q - kALoads) .., then the A scales of rows kARows wave ..
// + kARows, then the B scales
// (per column: of columns kBRows wave .. + kBRows; 128x128: the two column-block scales, by wave
// 0). `on` (wave-uniform) false: the load is issued with no lane enabled, so nothing is read or
// written. Every offset is the lane's offset in the load's resource (a position in the tensor, or
// kOob for a scale outside it) plus this K-block's advance.
template <bool PER_COL, int BM, int WM>
__device__ __forceinline__ void issue_load(int q, const Ops& op, uint32_t stage_base, int64_t kb, int wave,
                                           bool on = true) {
    using C = Cfg<BM, WM>;
    const uint32_t k = geom::fast_operand_advance(kb);
    const uint64_t all = on ? ~0ull : 0ull;
    const uint64_t half = on ? 0xFFFFFFFFull : 0ull;
    const uint64_t a_rows = on ? (C::kARows == 32 ? 0xFFFFFFFFull : 0xFFFFull) : 0ull;
    if (q < C::kALoads) {
        dma16(stage_base + (C::kStageA + (C::kARows * wave + 8 * q) * 8) * 16, op.a[q], op.a_lane[q & 1] + k, all);
    } else if (q < C::kALoads + C::kBLoads) {
        const int qb = q - C::kALoads;
        dma16(stage_base + (C::kStageB + (C::kBRows * wave + 8 * qb) * 8) * 16, op.b[qb & 3],
              op.b_lane[(qb & 1) + 2 * (qb >> 2)] + k, all);
    } else if (q == C::kALoads + C::kBLoads) {
        dma4(stage_base + C::kStageSA * 16 + 4 * C::kARows * wave, op.as,
             op.as_base + static_cast<uint32_t>(kb * op.as_step), a_rows);
    } else if (PER_COL) {
        dma4(stage_base + C::kStageSB * 16 + 4 * C::kBRows * wave, op.bs,
             op.bs_base + static_cast<uint32_t>(kb * op.bs_step), C::kBRows == 64 ? all : half);
    } else {
        dma4(stage_base + C::kStageSB * 16, op.bs, op.bs_base + static_cast<uint32_t>(kb * op.bs_step),
             on && wave == 0 ? 0x3ull : 0ull);
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

template <bool PER_COL, int GROUP, int BM, int WM = kWM>
__global__ __launch_bounds__((Cfg<BM, WM>::kThreads), 1) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s,
    const uint8_t* __restrict__ B, int64_t ldb, const float* __restrict__ b_s, int64_t bs_nb,
    int64_t bs_kb, uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K, int mt,
    int nt, int c_vec, Grouping grp) {
    using Cf = Cfg<BM, WM>;
    constexpr int kStageA = Cf::kStageA, kStageB = Cf::kStageB, kStageSA = Cf::kStageSA, kStageSB = Cf::kStageSB;
    constexpr int kStageSize = Cf::kStageSize, kLoads = Cf::kLoads;
    constexpr int kMSub = Cf::kMSub;
    __shared__ u32x4 smem[kStages * kStageSize];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % Cf::kWavesM;  // rows WM wm .. of the tile
    const int wn = wave / Cf::kWavesM;  // columns 128 wn .. of the tile
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    int tm, tn;
    geom::tile_of(blockIdx.x, mt, nt, tm, tn);
    int64_t m0 = static_cast<int64_t>(tm) * BM;  // this tile's rows are [m0, min(m0 + BM, m_end))
    int64_t m_end = M;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    // K-blocks (the last one may be partial: only for the ungrouped GEMMs, whose callers allow it)
    int64_t Kb = (K + kGroup - 1) / kGroup;
    bool unaligned = false;  // kGroupK: an expert range off the 128 grid (its C becomes NaN)
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
            const int64_t tiles = (b - a + BM - 1) / BM;
            if (tm < first + tiles) {
                e = j;
                lo = a;
                hi = b;
                break;
            }
            first += tiles;
        }
        if (e < 0) return;  // a spare workgroup of the grid's upper bound: the whole group leaves
        m0 = lo + (tm - first) * BM;
        m_end = hi;
        B += e * grp.b_stride;
        b_s += e * grp.bs_stride;
    } else if (GROUP == kGroupK) {
        // expert e = blockIdx.y owns the K-blocks [offsets[e] / 128, offsets[e + 1] / 128) of A and B
        // (token ranges of the weight gradient, multiples of 128) and writes its own C. A range
        // whose ends (clamped into [0, K] and to non-decreasing order) are not multiples of 128 has
        // no K-blocks of its own: its C is filled with NaN and *status set, nothing is rounded.
        // Up to 64 experts, blockIdx.y = r runs the expert of rank r in decreasing order of K-blocks
        // (ties by index): workgroups are dispatched in order of blockIdx.y, so the longest tiles
        // start first and the shortest fill the last round.
        int64_t e = blockIdx.y;
        if (grp.E <= 64) {
            const auto kblocks = [&](int64_t j) -> int64_t {
                const int64_t a = min(max(grp.offsets[j], int64_t{0}), K);
                const int64_t b = min(max(grp.offsets[j + 1], a), K);
                return a % kGroup != 0 || b % kGroup != 0 ? 0 : b / kGroup - a / kGroup;
            };
            const int64_t mine = lane < grp.E ? kblocks(lane) : -1;  // lane j: expert j's K-blocks
            int rank = 0;
            for (int j = 0; j < static_cast<int>(grp.E); ++j) {
                const uint32_t lo32 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine), j));
                const uint32_t hi32 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine >> 32), j));
                const int64_t kj = static_cast<int64_t>((static_cast<uint64_t>(hi32) << 32) | lo32);
                rank += kj > mine || (kj == mine && j < lane) ? 1 : 0;
            }
            const uint64_t hit = __ballot(lane < grp.E && rank == static_cast<int>(blockIdx.y));
            if (hit != 0) e = __ffsll(static_cast<unsigned long long>(hit)) - 1;  // ranks are a permutation: one lane
        }
        const int64_t lo = min(max(grp.offsets[e], int64_t{0}), K);
        const int64_t hi = min(max(grp.offsets[e + 1], lo), K);
        const int64_t kb0 = lo / kGroup;
        Kb = hi / kGroup - kb0;
        if (lo % kGroup != 0 || hi % kGroup != 0) {
            Kb = 0;
            unaligned = true;
            if (grp.status != nullptr && blockIdx.x == 0 && tid == 0) *grp.status = 1;
        }
        A += kb0 * kGroup;
        B += kb0 * kGroup;
        a_s += kb0 * M;
        b_s += PER_COL ? kb0 * N : kb0 * bs_kb;
        C += e * grp.c_stride;
    } else if (GROUP == kSplitK) {
        // slice s owns K-blocks [kb0, kb1) of the whole K and stops at K in the last one
        const int64_t KbT = Kb;
        const int64_t kb0 = geom::split_begin(KbT, gridDim.y, blockIdx.y);
        const int64_t kb1 = geom::split_begin(KbT, gridDim.y, blockIdx.y + 1);
        Kb = kb1 - kb0;
        K = min(K, kb1 * kGroup) - kb0 * kGroup;
        A += kb0 * kGroup;
        B += kb0 * kGroup;
        a_s += kb0 * M;
        b_s += PER_COL ? kb0 * N : kb0 * bs_kb;
    }

    Ops op;
    {
        const int64_t arows = (m_end - m0) < BM ? (m_end - m0) : BM;
        const int64_t brows = (N - n0) < kBN ? (N - n0) : kBN;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            op.a[q] = make_rsrc(A + (m0 + geom::fast_operand_first_row(q)) * lda, geom::fast_operand_range(q, arows, lda));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            op.b[q] = make_rsrc(B + (n0 + geom::fast_operand_first_row(q)) * ldb, geom::fast_operand_range(q, brows, ldb));
        op.as = make_rsrc(a_s, M * Kb * 4);
        op.bs = make_rsrc(b_s, PER_COL ? N * Kb * 4 : 4 * geom::bscale_blk_extent(N, Kb, bs_nb, bs_kb));
#pragma unroll
        for (int par = 0; par < 2; ++par) op.a_lane[par] = geom::fast_operand_lane(Cf::kARows, wave, par, lane, lda);
#pragma unroll
        for (int v = 0; v < (Cf::kBLoads > 4 ? 4 : 2); ++v)
            op.b_lane[v] = geom::fast_operand_lane(Cf::kBRows, wave, (v & 1) + 4 * (v >> 1), lane, ldb);
        op.as_base = geom::fast_ascale_base(Cf::kARows, m0, m_end, wave, lane);
        op.as_step = 4 * M;
        if (PER_COL) {
            op.bs_base = geom::fast_bscale_col_base(Cf::kBRows, n0, N, wave, lane);
            op.bs_step = 4 * N;
        } else {
            op.bs_base = geom::fast_bscale_blk_base(tn, N, bs_nb, wave, lane);
            op.bs_step = 4 * bs_kb;
        }
        op.lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)));
    }

    v4f acc[kMSub][kNSub];
    const float acc0 = unaligned ? __builtin_nanf("") : 0.0f;
#pragma unroll
    for (int i = 0; i < kMSub; ++i)
#pragma unroll
        for (int j = 0; j < kNSub; ++j) acc[i][j] = v4f{acc0, acc0, acc0, acc0};

    if (Kb > 0) {
        auto stage_base = [&](int stage) { return op.lds + static_cast<uint32_t>(stage * kStageSize * 16); };
        // Fragment lane (l16, lg) holds 16-byte chunks lg and lg + 4 of its row (row bytes
        // [16 lg, 16 lg + 16) and [64 + 16 lg, 64 + 16 lg + 16)). Any assignment of a row's 128
        // bytes to the four lane groups' 32 operand bytes gives the same dot product as long as A
        // and B use the same one; this one makes every ds_read_b128 conflict free at the full LDS
        // rate (4 cycles per instruction on gfx950, where chunks 2 lg and 2 lg + 1 take 8).
        const int sw = geom::lds_swizzle(l16);  // the same for every fragment row 16 x + l16
        const int pos_lo = lg ^ sw;
        const int pos_hi = (lg + 4) ^ sw;

        // prologue: block 0 into stage 0
#pragma unroll
        for (int q = 0; q < kLoads; ++q) issue_load<PER_COL, BM, WM>(q, op, stage_base(0), 0, wave);
        wait_own_loads<0>();

        // Bytes of the last K-block that lie below K (128 when K % 128 == 0). Its loads read whole
        // 128-byte rows, so bytes at and past K (row padding, or the start of the next row) are
        // zeroed in the fragment registers of that block (geom::tail_keep_mask).
        const int krem = static_cast<int>(K - (Kb - 1) * kGroup);
        const bool partial = krem != kGroup;
        auto tail_mask = [&](v8i v) {
#pragma unroll
            for (int d = 0; d < 8; ++d) v[d] = static_cast<int>(static_cast<uint32_t>(v[d]) & geom::tail_keep_mask(krem, lg, d));
            return v;
        };

        // block 0 is visible to every wave; block 1 goes into stage 1
        lds_barrier();
        if (Kb > 1) {
#pragma unroll
            for (int q = 0; q < kLoads; ++q) issue_load<PER_COL, BM, WM>(q, op, stage_base(1), 1, wave);
        }

        auto read_a = [&](const u32x4* st, int i, bool tail) {
            const int r = WM * wm + 16 * i + l16;
            const v8i v = to_v8i(st[kStageA + r * 8 + pos_lo], st[kStageA + r * 8 + pos_hi]);
            return tail ? tail_mask(v) : v;
        };
        auto read_b = [&](const u32x4* st, int j, bool tail) {
            const int r = 128 * wn + 16 * j + l16;
            const v8i v = to_v8i(st[kStageB + r * 8 + pos_lo], st[kStageB + r * 8 + pos_hi]);
            return tail ? tail_mask(v) : v;
        };
        // per-column B scales of subtile j (four consecutive columns per lane)
        auto read_bsj = [&](const u32x4* st, int j) {
            const float* sbs = reinterpret_cast<const float*>(st + kStageSB) + 128 * wn;
            return PER_COL ? *reinterpret_cast<const v4f*>(sbs + 16 * j + 4 * lg) : v4f{1.0f, 1.0f, 1.0f, 1.0f};
        };
        // the factor a_s[m, kb] (times the 128x128 B scale of the wave's column block) of each of
        // the lane's four rows
        auto read_factors = [&](const u32x4* st, float (&fo)[kMSub]) {
            const float* sa = reinterpret_cast<const float*>(st + kStageSA) + WM * wm;
            const float bsc = PER_COL ? 1.0f : reinterpret_cast<const float*>(st + kStageSB)[wn];
#pragma unroll
            for (int i = 0; i < kMSub; ++i) fo[i] = PER_COL ? sa[16 * i + l16] : sa[16 * i + l16] * bsc;
        };

        // Carried from one K-block to the next: the block's A fragments, its B fragments in a
        // four-deep ring (subtile j in bf[j % 4], read two subtiles ahead of its MFMAs), its
        // factors, and the partials of its last subtile column with their factors (rescaled just
        // before the next block's first MFMAs overwrite them).
        v8i af[kMSub];
        v8i bf[4];
        float f[kMSub];
        v4f pp[kMSub];
        v4f bsj_prev = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < kMSub; ++i) {
            af[i] = read_a(smem, i, false);
            f[i] = 0.0f;
            pp[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};  // a zero partial with a zero factor adds +0
        }
        bf[0] = read_b(smem, 0, false);
        bf[1] = read_b(smem, 1, false);

        // partial of subtile (i, j) times its factors, into the totals
        auto rescale = [&](int i, int j, const v4f& p, const float (&fi)[kMSub], const v4f& bsj) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[i][j][e] = fmaf(p[e], PER_COL ? fi[i] * bsj[e] : fi[i], acc[i][j][e]);
        };

        // One K-block. Subtile columns 0..5 run on fragments read from this block's stage; before
        // column 6 every fragment and scale of the block has been read, so one barrier there
        // (after each wave's wait for its own loads of block kb+1) both publishes block kb+1 and
        // frees this block's stage. Block kb+2 is then loaded into it -- four of the wave's loads
        // right away, the rest two per column over the next block's first columns, so the memory
        // system never sees a whole block requested at once -- and block kb+1's first fragments
        // are read while columns 6 and 7 keep the matrix cores busy; its A fragments replace this
        // block's right after their last MFMA. TAIL: the partial last K-block, whose fragments are
        // read again masked and which prefetches nothing. One body serves both stages (the stage
        // index is a run-time value: a body unrolled per stage makes the allocator spill).
        auto body = [&](int64_t kb, auto tail_tag) {
            constexpr bool TAIL = decltype(tail_tag)::value;
            const int cur = static_cast<int>(kb & 1);
            const u32x4* st = smem + cur * kStageSize;
            const u32x4* stn = smem + (cur ^ 1) * kStageSize;
            v4f bsj6 = {1.0f, 1.0f, 1.0f, 1.0f}, bsj7 = {1.0f, 1.0f, 1.0f, 1.0f};
            if (TAIL) {
#pragma unroll
                for (int i = 0; i < kMSub; ++i) af[i] = read_a(st, i, true);
                bf[0] = read_b(st, 0, true);
                bf[1] = read_b(st, 1, true);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kNSub; ++j) {
                if (j == 6 && !TAIL) {
                    wait_own_loads<0>();  // this wave's loads of block kb+1 have landed
                    lds_barrier();        // ... every wave's; no wave reads stage cur any more
                    // block kb+2 into this block's stage (none past the last block): loads 0..3 now,
                    // the rest over the next block's first columns
                    const bool more = kb + 2 < Kb;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        issue_load<PER_COL, BM, WM>(q, op, stage_base(cur), more ? kb + 2 : kb, wave, more);
                    // slots 0 and 1 were last used by subtiles 4 and 5
                    bf[0] = read_b(stn, 0, false);
                    bf[1] = read_b(stn, 1, false);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (!TAIL && j < Cf::kPendCols) {
                    // the rest of block kb+1's loads (its first four were issued by the previous
                    // block after its barrier; block 0 issues none, the prologue loaded block 1)
                    const bool pend = kb >= 1 && kb + 1 < Kb;
                    const int64_t pkb = pend ? kb + 1 : kb;
                    if (4 + 2 * j < kLoads) issue_load<PER_COL, BM, WM>(4 + 2 * j, op, stage_base(cur ^ 1), pkb, wave, pend);
                    if (5 + 2 * j < kLoads) issue_load<PER_COL, BM, WM>(5 + 2 * j, op, stage_base(cur ^ 1), pkb, wave, pend);
                }
                if (j + 2 < kNSub) bf[(j + 2) % 4] = read_b(st, j + 2, TAIL);
                v4f bsj;
                if (j < 6) {
                    bsj = read_bsj(st, j);
                    if (j == 5) {
                        bsj6 = read_bsj(st, 6);
                        bsj7 = read_bsj(st, 7);
                    }
                } else {
                    bsj = j == 6 ? bsj6 : bsj7;
                }
                // the partial pp[i] holds (subtile (i, j-1); at j = 0 the previous block's (i, 7))
                // is rescaled just before the MFMA that overwrites it
#pragma unroll
                for (int i = 0; i < kMSub; ++i) {
                    rescale(i, j == 0 ? kNSub - 1 : j - 1, pp[i], f, bsj_prev);
                    pp[i] = mfma_fp8_16x16x128(bf[j % 4], af[i]);
                    if (j == kNSub - 1 && !TAIL) af[i] = read_a(stn, i, false);
                }
                // this block's factors, once the previous block's last partials are rescaled
                if (j == 0) read_factors(st, f);
                bsj_prev = bsj;
                if (j + 2 < kNSub) __builtin_amdgcn_sched_group_barrier(0x100, PER_COL ? 3 : 2, 0);
                if (PER_COL && j == 5) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < kMSub; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x002, PER_COL ? 8 : 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (j == kNSub - 1 && !TAIL) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        const int64_t Kb_full = partial ? Kb - 1 : Kb;
        for (int64_t kb = 0; kb < Kb_full; ++kb) body(kb, std::false_type{});
        if (partial) body(Kb - 1, std::true_type{});
        // the last block's last subtile column
#pragma unroll
        for (int i = 0; i < kMSub; ++i) rescale(i, kNSub - 1, pp[i], f, bsj_prev);
        wait_own_loads<0>();
    }

    if constexpr (GROUP == kSplitK) {
        // fp32 partial tile of this K slice, straight from the totals: 16 bytes per lane
        float* P = reinterpret_cast<float*>(C) + static_cast<int64_t>(blockIdx.y) * grp.c_stride;
#pragma unroll
        for (int i = 0; i < kMSub; ++i) {
            const int64_t m = geom::fast_partial_row(WM, m0, wm, i, lane);
            if (m >= m_end) continue;
#pragma unroll
            for (int j = 0; j < kNSub; ++j) {
                const int64_t n = geom::fast_partial_col(n0, wn, j, lane);
                if (n < N) *reinterpret_cast<v4f*>(P + m * ldc + n) = acc[i][j];
            }
        }
        return;
    }

    // Epilogue: each wave's 64 x 128 bf16 block goes through LDS (the stages are free once every
    // wave has left the K-loop), so the global stores are 16 bytes per lane and whole 128-byte
    // lines (a lane's own outputs are 4 columns of one row). Row r of a block holds 16 chunks of 16
    // bytes, chunk c at position c ^ (r % 16), which keeps both LDS passes free of bank conflicts.
    __syncthreads();
    uint8_t* cblk = reinterpret_cast<uint8_t*>(smem) + wave * (WM * kWN * 2);
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
    for (int p = 0; p < WM / 4; ++p) {
        const int r = 4 * p + (lane >> 4);
        const u32x4 v = *reinterpret_cast<const u32x4*>(cblk + r * 256 + ((cc ^ (r & 15)) * 16));
        const int64_t m = geom::fast_store_row(WM, m0, wm, p, lane);
        if (m >= m_end) continue;
        const int64_t n = geom::fast_store_col(n0, wn, lane);
        uint16_t* dst = C + m * ldc + n;
        if (c_vec && n + 8 <= N) {
            // streaming store: the output is not read again by this kernel, and lines that stay
            // dirty in L2 would all be written back at the end of the launch
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
        } else {
            const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// C[m, n] = bf16(sum over the S partial tiles of fp32 P[s][m][n]), slices summed in order 0 .. S-1.
// Thread work item: 8 consecutive columns of one row (the partial rows are padded to a multiple
// of 8 floats).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ P, int64_t ldp,
                                                           int64_t slice, int S, uint16_t* __restrict__ C,
                                                           int64_t ldc, int64_t M, int64_t N, int c_vec) {
    const int64_t chunks = (N + 7) / 8;
    const int64_t total = M * chunks;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t m = t / chunks;
        const int64_t n = (t - m * chunks) * 8;
        const float* p = P + m * ldp + n;
        v4f s0 = *reinterpret_cast<const v4f*>(p);
        v4f s1 = *reinterpret_cast<const v4f*>(p + 4);
        for (int s = 1; s < S; ++s) {
            s0 += *reinterpret_cast<const v4f*>(p + s * slice);
            s1 += *reinterpret_cast<const v4f*>(p + s * slice + 4);
        }
        const uint32_t w[4] = {pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]), pack_bf16x2(s1[0], s1[1]),
                               pack_bf16x2(s1[2], s1[3])};
        uint16_t* dst = C + m * ldc + n;
        if (c_vec && n + 8 <= N) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace fast

// ==============================================================================================
// Thin kernel: 64 x BN tiles (BN = 32, 64 or 128) of 4 waves (2 x 2, each 32 x BN/2) or, for BN >= 64
// when the grid is at most one workgroup per CU, 8 waves (4 x 2, each 16 x BN/2), for problems
// whose 128-row tiles of the fast kernel would fill at most half the CUs (few rows: the short-and-
// wide GEMMs), every tile over the whole K range: no partial tiles to sum. With one or two such
// workgroups per CU the K-loop is bound by latency (waits, barriers, LDS reads, the MFMA -> FMA
// chains), not by the matrix cores or memory, so the pipeline is deep (STAGES = 2 .. 12 LDS
// stages) and an iteration multiplies one, two or four K-blocks behind one workgroup barrier
// (geometry.hpp: thin_blocks_per_step, thin_ahead, thin_wait_later; the CPU check simulates it).
// Each K-block's A and B rows go global -> LDS by the fast kernel's direct loads and LDS swizzle; a
// wave multiplies its 2 x BN/32 subtiles and rescales each partial into its totals exactly as the
// fast kernel does, so the two kernels give bit-identical results.
namespace thin {

// W waves per workgroup: 4 (2 x 2, each 32 x BN/2) or, for BN >= 64, 8 (4 x 2, each 16 x BN/2).
template <int BN, bool PER_COL, int W>
struct TCfg {
    static_assert(W == 4 || (W == 8 && BN >= 64), "8-wave thin tiles are 64 or 128 columns wide");
    static constexpr int kMS = 8 / W;    // 16-row subtiles per wave
    static constexpr int kNS = BN / 32;  // 16-column subtiles per wave
    static constexpr int kLoads = (geom::kThinBM + BN) / (8 * W);
    // LDS image of one stage (16-byte units): A rows 0..63, B rows 0..BN-1, the 64 A scales, the B
    // scales (per column: BN floats; 128x128: one float)
    static constexpr int kStageA = 0;
    static constexpr int kStageB = geom::kThinBM * 8;
    static constexpr int kStageSA = kStageB + BN * 8;
    static constexpr int kStageSB = kStageSA + geom::kThinBM / 4;
    static constexpr int kStageSize = kStageSB + (PER_COL ? BN / 4 : 1);
    static_assert(kStageSize == geom::thin_stage_units(BN, PER_COL), "stage size as the schedule counts it");
};

// Wait until this wave's loads of the block being multiplied have landed: `later` (0..MAXL)
// blocks issued after it are still allowed in flight, L instructions each (vmcnt is 6 bits wide).
template <int L, int MAXL>
__device__ __forceinline__ void wait_block(int later) {
    static_assert(L * MAXL <= 63, "outstanding loads beyond the vmcnt range");
    if constexpr (MAXL == 0) {
        fast::wait_own_loads<0>();
    } else {
        if (later >= MAXL) fast::wait_own_loads<L * MAXL>();
        else wait_block<L, MAXL - 1>(later);
    }
}

template <bool PER_COL, int BN, int STAGES, int W>
__global__ __launch_bounds__(64 * W) void gemm_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const float* __restrict__ a_s, const uint8_t* __restrict__ B,
    int64_t ldb, const float* __restrict__ b_s, int64_t bs_nb, int64_t bs_kb, uint16_t* __restrict__ C,
    int64_t ldc, int64_t M, int64_t N, int64_t K, int mt, int nt, int c_vec) {
    using T = TCfg<BN, PER_COL, W>;
    static_assert(STAGES >= 2 && STAGES * T::kStageSize * 16 <= sched::kLdsPerCu, "stages beyond the LDS");
    constexpr int kMS = T::kMS, kNS = T::kNS, kLoads = T::kLoads;
    __shared__ u32x4 smem[STAGES * T::kStageSize];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % (W / 2);  // rows thin_rows_per_wave(W) wm .. of the tile
    const int wn = wave / (W / 2);  // columns (BN / 2) wn .. of the tile
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    int tm, tn;
    geom::tile_of(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * geom::kThinBM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;
    // K-blocks as int: K <= ld <= 2^23 (the C ABI's operand bound)
    const int Kb = static_cast<int>((K + kGroup - 1) / kGroup);

    const int64_t arows = (M - m0) < geom::kThinBM ? (M - m0) : geom::kThinBM;
    const int64_t brows = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + m0 * lda, geom::thin_operand_range(arows, lda));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + n0 * ldb, geom::thin_operand_range(brows, ldb));
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_s, M * Kb * 4);
    const __amdgpu_buffer_rsrc_t rbs =
        make_rsrc(b_s, PER_COL ? N * Kb * 4 : 4 * geom::bscale_blk_extent(N, Kb, bs_nb, bs_kb));
    uint32_t lane_off[kLoads], unit[kLoads];
    bool is_a[kLoads];
#pragma unroll
    for (int p = 0; p < kLoads; ++p) {
        is_a[p] = geom::thin_load_is_a(BN, W, wave, p);
        lane_off[p] = geom::thin_operand_lane(geom::thin_group(BN, W, wave, p), lane, is_a[p] ? lda : ldb);
        unit[p] = static_cast<uint32_t>(geom::thin_load_unit(BN, W, wave, p));
    }
    const bool b_scales = geom::thin_has_bscale_load(BN, PER_COL, wave);
    const uint32_t as_base = geom::thin_ascale_base(m0, M, lane);
    const uint32_t bs_base = PER_COL ? geom::thin_bscale_col_base(BN, n0, N, wave, lane)
                                     : geom::thin_bscale_blk_base(n0, bs_nb, lane);
    const int64_t bs_step = PER_COL ? 4 * N : 4 * bs_kb;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem)));
    const uint64_t bs_lanes = geom::thin_bscale_lanes(BN, PER_COL);

    // K-block kb into stage s: the wave's operand groups, then its scale load (wave 0: A scales;
    // waves 3 and, per column at BN = 128, 2: B scales)
    auto issue = [&](int kb, int s) {
        const uint32_t base = lds0 + static_cast<uint32_t>(s * T::kStageSize * 16);
        const uint32_t adv = geom::fast_operand_advance(kb);
#pragma unroll
        for (int p = 0; p < kLoads; ++p) fast::dma16(base + unit[p] * 16, is_a[p] ? ra : rb, lane_off[p] + adv, ~0ull);
        if (wave == 0)
            fast::dma4(base + T::kStageSA * 16, ras, as_base + geom::fast_ascale_advance(kb, M), ~0ull);
        else if (b_scales)
            fast::dma4(base + T::kStageSB * 16 + (wave == 2 ? 256 : 0), rbs,
                       bs_base + static_cast<uint32_t>(kb * bs_step), bs_lanes);
    };

    v4f acc[kMS][kNS];
#pragma unroll
    for (int i = 0; i < kMS; ++i)
#pragma unroll
        for (int j = 0; j < kNS; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Fragment lane (l16, lg) holds 16-byte chunks lg and lg + 4 of its row, as in the fast kernel;
    // the bytes of a partial last K-block at and past K are zeroed in the fragment registers.
    const int sw = geom::lds_swizzle(l16);
    const int pos_lo = lg ^ sw;
    const int pos_hi = (lg + 4) ^ sw;
    const int krem = static_cast<int>(K - static_cast<int64_t>(Kb - 1) * kGroup);
    const bool scale_wave = wave == 0 || b_scales;

    // K-block kb lives in stage kb % STAGES. An iteration multiplies NB consecutive blocks (four
    // from twelve stages on, two from four, else one) behind one barrier: it waits for its blocks
    // (AHEAD - NB later ones may stay in flight), passes the barrier (after which no wave reads the
    // stages of the previous iteration's blocks), issues the NB blocks AHEAD = STAGES - NB after its
    // first into those stages, and multiplies. At the start of the iteration for block kb, blocks
    // through kb + AHEAD - 1 have been issued.
    constexpr int NB = geom::thin_blocks_per_step(STAGES);
    constexpr int AHEAD = geom::thin_ahead(STAGES);
#pragma unroll
    for (int s = 0; s < AHEAD; ++s)
        if (s < Kb) issue(s, geom::thin_stage_of(STAGES, s));

    // One K-block's products. TAIL: the partial last block, whose fragment bytes at and past K are
    // zeroed (a second instance, so the full blocks carry no per-fragment branch).
    auto compute = [&](int kb, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const u32x4* st = smem + geom::thin_stage_of(STAGES, kb) * T::kStageSize;
        auto frag = [&](int unit) {
            v8i v = to_v8i(st[unit + pos_lo], st[unit + pos_hi]);
            if (TAIL) {
#pragma unroll
                for (int d = 0; d < 8; ++d) v[d] = static_cast<int>(static_cast<uint32_t>(v[d]) & geom::tail_keep_mask(krem, lg, d));
            }
            return v;
        };
        v8i af[kMS], bf[kNS];
        float fa[kMS];
        const float* sa = reinterpret_cast<const float*>(st + T::kStageSA);
        const float* sb = reinterpret_cast<const float*>(st + T::kStageSB);
#pragma unroll
        for (int i = 0; i < kMS; ++i) {
            const int r = geom::thin_rows_per_wave(W) * wm + 16 * i + l16;
            af[i] = frag(T::kStageA + r * 8);
            fa[i] = PER_COL ? sa[r] : sa[r] * sb[0];
        }
#pragma unroll
        for (int j = 0; j < kNS; ++j) bf[j] = frag(T::kStageB + ((BN / 2) * wn + 16 * j + l16) * 8);
#pragma unroll
        for (int j = 0; j < kNS; ++j) {
            const v4f bsj = PER_COL ? *reinterpret_cast<const v4f*>(sb + (BN / 2) * wn + 16 * j + 4 * lg)
                                    : v4f{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
            for (int i = 0; i < kMS; ++i) {
                const v4f p = mfma_fp8_16x16x128(bf[j], af[i]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] = fmaf(p[e], PER_COL ? fa[i] * bsj[e] : fa[i], acc[i][j][e]);
            }
        }
    };
    // Blocks kb .. kb + n - 1 (n <= NB) have landed for every wave, then the next n are issued;
    // the blocks kb + n .. kb + AHEAD - 1 may stay in flight.
    auto step = [&](int kb, int n) {
        const int later = geom::thin_wait_later(STAGES, kb, n, Kb);
        if (scale_wave) wait_block<kLoads + 1, AHEAD - 1>(later);
        else wait_block<kLoads, AHEAD - 1>(later);
        fast::lds_barrier();
        for (int q = 0; q < n; ++q)
            if (kb + AHEAD + q < Kb) issue(kb + AHEAD + q, geom::thin_stage_of(STAGES, kb + AHEAD + q));
    };
    const int Kb_full = krem != kGroup ? Kb - 1 : Kb;
    int kb = 0;
    for (; kb + NB <= Kb_full; kb += NB) {
        step(kb, NB);
#pragma unroll
        for (int q = 0; q < NB; ++q) compute(kb + q, std::false_type{});
    }
    for (; kb < Kb_full; ++kb) {
        step(kb, 1);
        compute(kb, std::false_type{});
    }
    if (Kb_full < Kb) {
        step(Kb - 1, 1);
        compute(Kb - 1, std::true_type{});
    }

    // bf16 outputs straight from the totals: a lane's four consecutive columns of one row
#pragma unroll
    for (int i = 0; i < kMS; ++i) {
        const int64_t m = geom::thin_store_row(m0, W, wm, i, lane);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < kNS; ++j) {
            const int64_t n = geom::thin_store_col(n0, BN, wn, j, lane);
            uint16_t* dst = C + m * ldc + n;
            const uint32_t w0 = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
            const uint32_t w1 = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
            if (c_vec && n + 4 <= N) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
            } else {
                const uint32_t w[2] = {w0, w1};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

}  // namespace thin

}  // namespace

// Scratch of the allocation-free GEMM entry point: the split-K partial tiles, in a file-scope device
// array (each GPU holds its own copy for the life of the process). In host code the array's name is
// a stand-in, not a device address: host code uses only the address hipGetSymbolAddress returns for
// the current device, looked up on the first use on that device and kept. 64 MiB covers every plan
// gemm_split_plan makes (at most one slice per CU of a 256 x 256 fp32 tile: 256 x 256 KiB).
constexpr int64_t kScratchBytes = 64LL << 20;
static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {
std::mutex g_scratch_mutex;
float* g_scratch_ptr[64];
}  // namespace

int64_t gemm_scratch_bytes() { return kScratchBytes; }

hipError_t gemm_scratch(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// The schedule (tile shape, K split, thin pipeline depth) is in schedule.hpp.

namespace {

// The fast kernel with tile height BM, unsplit or split over plan.S slices.
template <int BM, int WM>
hipError_t launch_fast(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b, int64_t ldb,
                       BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       const SplitPlan& plan, float* workspace, int cus, hipStream_t stream) {
    constexpr int kThreads = fast::Cfg<BM, WM>::kThreads;
    const int64_t mt = (M + BM - 1) / BM;
    const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const int64_t nb = bs.per_column ? 0 : bs.stride_nb;
    const int64_t kbs = bs.per_column ? 0 : bs.stride_kb;
    if (plan.S > 1) {
        // K split over plan.S workgroups per tile: fp32 partial tiles, then their sum in bf16
        if (workspace == nullptr) return hipErrorInvalidValue;
        const fast::Grouping g{nullptr, 0, 0, 0, M * plan.ldp, nullptr};
        const dim3 grid(static_cast<unsigned>(mt * nt), static_cast<unsigned>(plan.S));
        uint16_t* P = reinterpret_cast<uint16_t*>(workspace);
        if (bs.per_column)
            fast::gemm_kernel<true, fast::kSplitK, BM, WM><<<grid, kThreads, 0, stream>>>(
                a, lda, a_s, b, ldb, bs.ptr, nb, kbs, P, plan.ldp, M, N, K, (int)mt, (int)nt, 0, g);
        else
            fast::gemm_kernel<false, fast::kSplitK, BM, WM><<<grid, kThreads, 0, stream>>>(
                a, lda, a_s, b, ldb, bs.ptr, nb, kbs, P, plan.ldp, M, N, K, (int)mt, (int)nt, 0, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int c_vec16 = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
        const int64_t items = M * ((N + 7) / 8);
        int64_t wgs = (items + 255) / 256;
        if (wgs > static_cast<int64_t>(cus) * 8) wgs = static_cast<int64_t>(cus) * 8;
        fast::split_reduce_kernel<<<dim3(static_cast<unsigned>(wgs)), 256, 0, stream>>>(
            workspace, plan.ldp, M * plan.ldp, plan.S, c, ldc, M, N, c_vec16);
        return hipGetLastError();
    }
    const int c_vec16 = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
    const dim3 grid(static_cast<unsigned>(mt * nt));
    const fast::Grouping none{nullptr, 0, 0, 0, 0, nullptr};
    if (bs.per_column)
        fast::gemm_kernel<true, fast::kGroupNone, BM, WM><<<grid, kThreads, 0, stream>>>(
            a, lda, a_s, b, ldb, bs.ptr, nb, kbs, c, ldc, M, N, K, (int)mt, (int)nt, c_vec16, none);
    else
        fast::gemm_kernel<false, fast::kGroupNone, BM, WM><<<grid, kThreads, 0, stream>>>(
            a, lda, a_s, b, ldb, bs.ptr, nb, kbs, c, ldc, M, N, K, (int)mt, (int)nt, c_vec16, none);
    return hipGetLastError();
}

// The thin kernel with tile width BN (no split; every tile over the whole K range) and STAGES LDS
// stages (STAGES - 1 K-blocks in flight per workgroup).
template <int BN, int STAGES, int W>
hipError_t launch_thin_stages(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b, int64_t ldb,
                              BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int mt, int nt,
                              hipStream_t stream) {
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 8 == 0) && (ldc % 4 == 0);
    const dim3 grid(static_cast<unsigned>(mt) * static_cast<unsigned>(nt));
    if (bs.per_column)
        thin::gemm_kernel<true, BN, STAGES, W><<<grid, 64 * W, 0, stream>>>(
            a, lda, a_s, b, ldb, bs.ptr, 0, 0, c, ldc, M, N, K, mt, nt, c_vec);
    else
        thin::gemm_kernel<false, BN, STAGES, W><<<grid, 64 * W, 0, stream>>>(
            a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb, bs.stride_kb, c, ldc, M, N, K, mt, nt, c_vec);
    return hipGetLastError();
}

template <int BN, int W>
hipError_t launch_thin_waves(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b, int64_t ldb,
                             BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int mt, int nt,
                             int stages, hipStream_t stream) {
#define BSFP8_THIN(S) return launch_thin_stages<BN, (S), W>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, mt, nt, stream)
    switch (stages) {
        case 2: BSFP8_THIN(2);
        case 3: BSFP8_THIN(3);
        case 4: BSFP8_THIN(4);
        case 6: BSFP8_THIN(6);
        case 8: if constexpr (BN <= 64) { BSFP8_THIN(8); } break;
        case 12: if constexpr (BN <= 32) { BSFP8_THIN(12); } break;
        default: break;
    }
#undef BSFP8_THIN
    return hipErrorInvalidValue;
}

// The pipeline depth and the waves per workgroup: `stages` / `waves` when the plan forces them (a
// depth must be instantiated for BN and fit the LDS; 8 waves need BN >= 64), else
// sched::thin_stages / sched::thin_waves.
template <int BN>
hipError_t launch_thin(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b, int64_t ldb,
                       BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int cus,
                       int stages, int waves, hipStream_t stream) {
    const int64_t mt = (M + geom::kThinBM - 1) / geom::kThinBM;
    const int64_t nt = (N + BN - 1) / BN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    if (stages == 0) stages = sched::thin_stages(BN, bs.per_column != 0, mt * nt, cus);
    if (waves == 0) waves = sched::thin_waves(BN, mt * nt, cus);
    if (stages > sched::thin_max_stages(BN, bs.per_column != 0)) return hipErrorInvalidValue;
    if (waves == 8) {
        if constexpr (BN >= 64)
            return launch_thin_waves<BN, 8>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, (int)mt, (int)nt, stages, stream);
        return hipErrorInvalidValue;
    }
    if (waves != 4) return hipErrorInvalidValue;
    return launch_thin_waves<BN, 4>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, (int)mt, (int)nt, stages, stream);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                       int64_t ldb, BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N,
                       int64_t K, bool fnuz, const SplitPlan& plan, float* workspace, int cus,
                       hipStream_t stream) {
    if (!fnuz) {
        if (plan.bm == geom::kThinBM) {
            if (plan.bn == 128)
                return launch_thin<128>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, cus, plan.stages, plan.waves, stream);
            if (plan.bn == 64)
                return launch_thin<64>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, cus, plan.stages, plan.waves, stream);
            return launch_thin<32>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, cus, plan.stages, plan.waves, stream);
        }
        if (plan.bm == fast::kBMSmall)
            return launch_fast<fast::kBMSmall, fast::kWMSmall>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, plan, workspace, cus, stream);
        return launch_fast<fast::kBM, fast::kWM>(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, plan, workspace, cus, stream);
    }
    // float8_e4m3fnuz: general kernel
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 8 == 0) && (ldc % 4 == 0);
    const int64_t mt = (M + gen::kBM - 1) / gen::kBM;
    const int64_t nt = (N + gen::kBN - 1) / gen::kBN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(mt * nt));
    if (bs.per_column)
        gen::gemm_kernel<true><<<grid, gen::kThreads, 0, stream>>>(a, lda, a_s, b, ldb, bs.ptr, 0, 0, c, ldc, M,
                                                                   N, K, (int)mt, (int)nt, c_vec);
    else
        gen::gemm_kernel<false><<<grid, gen::kThreads, 0, stream>>>(a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb,
                                                                    bs.stride_kb, c, ldc, M, N, K, (int)mt,
                                                                    (int)nt, c_vec);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped_rows(const uint8_t* a, int64_t lda, const float* a_s,
                                    const uint8_t* b, int64_t ldb, int64_t b_stride, BScale bs,
                                    int64_t bs_stride, const int64_t* offsets, int64_t E,
                                    uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                    hipStream_t stream) {
    if (K % kGroup != 0) return hipErrorInvalidValue;
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0);
    // every expert's last row tile may be partial: at most ceil(M / 256) + E row tiles
    const int64_t mt = (M + fast::kBM - 1) / fast::kBM + E;
    const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
    if (mt * nt > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const fast::Grouping g{offsets, E, b_stride, bs_stride, 0, nullptr};
    fast::gemm_kernel<false, fast::kGroupRows, fast::kBM><<<dim3(static_cast<unsigned>(mt * nt)), fast::Cfg<fast::kBM>::kThreads, 0, stream>>>(
        a, lda, a_s, b, ldb, bs.ptr, bs.stride_nb, bs.stride_kb, c, ldc, M, N, K, (int)mt, (int)nt,
        c_vec, g);
    return hipGetLastError();
}

hipError_t launch_gemm_grouped_k(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                                 int64_t ldb, const float* b_s, const int64_t* offsets, int64_t E,
                                 uint16_t* c, int64_t ldc, int64_t c_stride, int64_t M, int64_t N,
                                 int64_t K, int32_t* status, hipStream_t stream) {
    if (K % kGroup != 0) return hipErrorInvalidValue;
    const int c_vec = (reinterpret_cast<uintptr_t>(c) % 16 == 0) && (ldc % 8 == 0) && (c_stride % 8 == 0);
    const int64_t mt = (M + fast::kBM - 1) / fast::kBM;
    const int64_t nt = (N + fast::kBN - 1) / fast::kBN;
    if (mt * nt > 0x7FFFFFFFLL || E > 65535) return hipErrorInvalidValue;
    const fast::Grouping g{offsets, E, 0, 0, c_stride, status};
    fast::gemm_kernel<true, fast::kGroupK, fast::kBM><<<dim3(static_cast<unsigned>(mt * nt), static_cast<unsigned>(E)), fast::Cfg<fast::kBM>::kThreads, 0, stream>>>(
        a, lda, a_s, b, ldb, b_s, 0, 0, c, ldc, M, N, K, (int)mt, (int)nt, c_vec, g);
    return hipGetLastError();
}

}  // namespace bsfp8
