// gfx950 group quantizers: bf16 -> float8_e4m3fn (or float8_e4m3fnuz) codes + fp32 scales.
//
//   quantize_lhs             1x128 groups along K (act_quant_lhs), scales column-major [M, Kb]
//   quantize_rhs             128x1 groups down each column (act_quant_rhs), codes written transposed
//   quantize_weight_128x128  128x128 blocks (weight_quant_rhs), optional transposed copy
//   quantize_lhs_and_rhs     the 1x128 and the transposed 128x1 outputs of one tensor, one read
//   quantize_lhs_and_weight  quantize_lhs(x) and quantize_weight_128x128(w) in one launch
//
// Operations as listed in the quantization-correctness table of "Enable blockwise FP8 dense
// training kernels on ROCm" (block_size 128); the column-major scale layout and the rule that a
// scale store of a row >= M must be dropped come from that page's root-cause comment.
//
// Every kernel is instantiated for both element formats (FNUZ = false: e4m3fn, FP8_MAX 448;
// true: e4m3fnuz, FP8_MAX 240); only the scale pair and the final code conversion differ.
//
// All are HBM-bound: every input byte is read once with 16-byte loads, all of a tile's loads are in
// flight before the first wait, every output byte is written once, 16-lane (1x128) or LDS (128x1,
// 128x128) max reductions run on data already in registers, and the transposing variants turn the
// tile around in LDS so global stores stay contiguous along the output rows. quantize_lhs on
// aligned rows (K % 16 == 0) works in row strips instead of tiles: a workgroup reads whole rows,
// encodes them into LDS and only then writes them, so its reads and its writes are each one long
// contiguous stream.
#include "device_common.hpp"
#include "geometry.hpp"
#include "launch.hpp"

namespace bsfp8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive bf16 of row r (of nrows, row stride ld) starting at column c, as 4 packed dwords
// (element 2d in the low half of dword d); rows >= nrows and columns >= ncols read as +0.
// VEC (16-byte aligned rows and ncols % 8 == 0, so a lane's 8 columns are all in range or all
// out): one 16-byte load with no branch around it -- an out-of-range lane loads from x[0] and
// keeps zeros -- so the loads of a whole tile are in flight together. (A load inside a per-lane
// branch is followed by a wait for it before the branch joins: one memory round trip per load.)
template <bool VEC>
__device__ __forceinline__ void load8_packed(const uint16_t* __restrict__ x, int64_t ld, int64_t r,
                                             int64_t nrows, int64_t c, int64_t ncols, uint32_t w[4]) {
    if (VEC) {
        const bool in = r < nrows && c < ncols;
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (in ? r * ld + c : 0)));
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = in ? v[d] : 0u;
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = 0u;
        if (r < nrows) {
            const uint16_t* row = x + r * ld;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = (c + 2 * d < ncols) ? row[c + 2 * d] : 0u;
                const uint32_t hi = (c + 2 * d + 1 < ncols) ? row[c + 2 * d + 1] : 0u;
                w[d] = lo | (hi << 16);
            }
        }
    }
}

// The same 8 values as fp32 (exact).
template <bool VEC>
__device__ __forceinline__ void load8(const uint16_t* __restrict__ x, int64_t ld, int64_t r, int64_t nrows,
                                      int64_t c, int64_t ncols, float f[8]) {
    uint32_t w[4];
    load8_packed<VEC>(x, ld, r, nrows, c, ncols, w);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f[2 * d] = bf16_lo(w[d]);
        f[2 * d + 1] = bf16_hi(w[d]);
    }
}

// Store 8 code bytes (w0 = bytes 0..3, w1 = bytes 4..7) at row[c ..]; bytes at columns >= ncols
// are not written. VEC (8-byte aligned rows, ncols % 8 == 0): one 8-byte store or none.
template <bool VEC>
__device__ __forceinline__ void store8(uint8_t* __restrict__ row, int64_t c, int64_t ncols,
                                       uint32_t w0, uint32_t w1) {
    if (VEC) {
        if (c < ncols) *reinterpret_cast<uint2*>(row + c) = make_uint2(w0, w1);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c + j < ncols)
                row[c + j] = static_cast<uint8_t>(((j < 4 ? w0 : w1) >> (8 * (j & 3))) & 0xFF);
    }
}

// Store 16 code bytes at row[c ..], masked at ncols. VEC (16-byte aligned rows, ncols % 16 == 0):
// one 16-byte store or none.
template <bool VEC>
__device__ __forceinline__ void store16(uint8_t* __restrict__ row, int64_t c, int64_t ncols,
                                        uint4 v) {
    if (VEC) {
        if (c < ncols) *reinterpret_cast<uint4*>(row + c) = v;
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (c + j < ncols)
                row[c + j] = static_cast<uint8_t>((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
    }
}

// ------------------------------------------------------------------------------------------
// 1x128: a 16-lane team owns one (row, K-block) group, 8 elements per lane. A unit of work is
// kLhsRows consecutive rows of one K-block, so its scale stores are one contiguous run of a
// column-major scale column. Units are numbered K-block fastest: the workgroups running at one
// time read neighbouring 256-byte pieces of the same rows, i.e. contiguous stretches of x, which
// keeps DRAM pages open (numbering them row block fastest cost 10-15% of the bandwidth). The grid
// holds at most kLhsWgPerCu workgroups per CU; each walks the units with stride gridDim.x.
constexpr int kLhsRowsPerTeam = 4;
constexpr int kLhsRows = 16 * kLhsRowsPerTeam;
constexpr int kLhsWgPerCu = 8;

template <bool FNUZ, bool VEC_X, bool VEC_Q>
__global__ __launch_bounds__(256) void quantize_lhs_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ a_s, int64_t Kb, int64_t units) {
    const int lane16 = threadIdx.x & 15;
    const int team = threadIdx.x >> 4;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    int64_t rb, kb;
    geom::lhs_unit(u, Kb, rb, kb);
    const int64_t c = kb * kGroup + lane16 * 8;

    uint32_t w[kLhsRowsPerTeam][4];  // packed bf16 pairs
#pragma unroll
    for (int r = 0; r < kLhsRowsPerTeam; ++r) load8_packed<VEC_X>(x, ldx, geom::lhs_row(rb, kLhsRowsPerTeam, r, team), M, c, K, w[r]);
    // every row is encoded before the first store: a store issued while loads are outstanding
    // makes the wait for the next row's load also wait for that store
    uint32_t code[kLhsRowsPerTeam][2];
    float scale[kLhsRowsPerTeam];
#pragma unroll
    for (int r = 0; r < kLhsRowsPerTeam; ++r) {
        uint32_t am = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) am = max(am, max((w[r][d] << 16) & 0x7FFFFFFFu, w[r][d] & 0x7FFF0000u));
        am = umax_row16(am);
        const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
        code[r][0] = encode4_in_range<FNUZ>(bf16_lo(w[r][0]) * g.m, bf16_hi(w[r][0]) * g.m,
                                            bf16_lo(w[r][1]) * g.m, bf16_hi(w[r][1]) * g.m);
        code[r][1] = encode4_in_range<FNUZ>(bf16_lo(w[r][2]) * g.m, bf16_hi(w[r][2]) * g.m,
                                            bf16_lo(w[r][3]) * g.m, bf16_hi(w[r][3]) * g.m);
        scale[r] = g.s;
    }
#pragma unroll
    for (int r = 0; r < kLhsRowsPerTeam; ++r) {
        const int64_t m = geom::lhs_row(rb, kLhsRowsPerTeam, r, team);
        if (geom::row_stored(m, M)) {  // rows >= M store neither codes nor scales
            store8<VEC_Q>(q + m * ldq, c, K, code[r][0], code[r][1]);
            if (lane16 == 0) a_s[geom::colmajor_index(kb, M, m)] = scale[r];
        }
    }
    }
}

// ------------------------------------------------------------------------------------------
// 1x128 in row strips (16-byte aligned rows, K % 16 == 0): a 512-thread workgroup reads a strip of
// whole rows (or a chunk of at most 32 K-blocks of them) -- NL 16-byte pieces per thread, all in
// flight together -- encodes it into LDS, and only then writes it: codes as 16-byte pieces of
// contiguous rows, scales as runs of consecutive rows of each column-major scale column. Each
// workgroup's reads and writes are long contiguous streams and its read and write phases do not
// interleave, which the HBM serves faster than the tile kernel's 256-byte pieces of many rows with
// loads and stores mixed (8192 x 4096: 17.4 against 19.5 us; 4096 x 4096: 8.7 against 10.7 us).
template <bool FNUZ, int NL>
__global__ __launch_bounds__(geom::kStripThreads) void quantize_lhs_strip_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ a_s, int64_t Kb, geom::StripShape sh) {
    constexpr int T = geom::kStripThreads;
    __shared__ uint2 codes[T * NL];      // the strip's codes, row-major [rows][128 g] bytes
    __shared__ float scl[T * NL / 16];   // its scales, row-major [rows][g]

    const int t = threadIdx.x;
    int64_t strip, chunk;
    geom::strip_unit(blockIdx.x, sh.chunks, strip, chunk);
    const int64_t m0 = strip * sh.rows, kb0 = chunk * sh.g, c0 = kb0 * kGroup;

    uint32_t w[NL][4];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        int64_t m, c;
        const bool in = geom::strip_piece(t + T * j, sh, m0, c0, M, K, m, c);
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (in ? m * ldx + c : 0)));
#pragma unroll
        for (int d = 0; d < 4; ++d) w[j][d] = in ? v[d] : 0u;
    }
    // pieces past the strip hold zeros; their codes and scales land in LDS slots nothing reads
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        uint32_t am = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) am = max(am, max((w[j][d] << 16) & 0x7FFFFFFFu, w[j][d] & 0x7FFF0000u));
        am = umax_row16(am);
        const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
        const int p = t + T * j;
        codes[p] = make_uint2(encode4_in_range<FNUZ>(bf16_lo(w[j][0]) * g.m, bf16_hi(w[j][0]) * g.m,
                                                     bf16_lo(w[j][1]) * g.m, bf16_hi(w[j][1]) * g.m),
                              encode4_in_range<FNUZ>(bf16_lo(w[j][2]) * g.m, bf16_hi(w[j][2]) * g.m,
                                                     bf16_lo(w[j][3]) * g.m, bf16_hi(w[j][3]) * g.m));
        if ((t & 15) == 0) scl[p >> 4] = g.s;
    }
    __syncthreads();
    const u32x4* cs = reinterpret_cast<const u32x4*>(codes);
#pragma unroll
    for (int i = 0; i < (NL + 1) / 2; ++i) {
        int64_t m, c;
        const int qi = t + T * i;
        if (geom::strip_out_piece(qi, sh, m0, c0, M, K, m, c))
            __builtin_nontemporal_store(cs[qi], reinterpret_cast<u32x4*>(q + m * ldq + c));
    }
    for (int i = t; i < sh.rows * sh.g; i += T) {
        int64_t kb, m;
        if (geom::strip_scale(i, sh, m0, kb0, M, Kb, kb, m))
            a_s[geom::colmajor_index(kb, M, m)] = scl[(i % sh.rows) * sh.g + i / sh.rows];
    }
}

// ------------------------------------------------------------------------------------------
// 128x1 with transposed output: a workgroup owns one K-block (128 rows) x 64 columns.
// Thread t loads 4 consecutive rows (4*(t/8) ..) x 8 columns (8*(t%8) ..); column maxima go
// through LDS; the 4 codes of a column form one dword of the transposed tile, which is then
// written out as 128 contiguous bytes per output row. Workgroup order (kb_fast): K-block fastest
// makes the workgroups running together write contiguous stretches of the qT rows; column chunk
// fastest makes them read whole rows of x. The first is faster once the grid needs more than one
// round of resident workgroups (8192 x 4096: 22.0 -> 19.9 us; 16384 x 5120: 57 -> 48.5 us), the
// second when every workgroup is resident at once (4096 x 4096: 10.8 against 11.7 us).
constexpr int kRhsCols = 64;
constexpr int kRhsWgPerCu = 8;

template <bool FNUZ, bool VEC_X, bool VEC_Q>
__global__ __launch_bounds__(256) void quantize_rhs_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t N, int64_t ldx,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ s, int kb_fast) {
    __shared__ uint32_t red[32][kRhsCols + 1];
    __shared__ float mult[kRhsCols];
    __shared__ uint4 tileT[kRhsCols * 8];  // [column][8 x 16-byte chunks], chunk index swizzled

    const int t = threadIdx.x;
    const int cg = t & 7;
    const int rq = t >> 3;
    const int64_t kb = kb_fast ? blockIdx.x : blockIdx.y;
    const int64_t k0 = kb * kGroup;
    const int64_t n0 = static_cast<int64_t>(kb_fast ? blockIdx.y : blockIdx.x) * kRhsCols;
    const int64_t col = n0 + cg * 8;

    float f[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        load8<VEC_X>(x, ldx, k0 + rq * 4 + i, K, col, N, f[i]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t am = max(max(abs_bits(f[0][j]), abs_bits(f[1][j])),
                          max(abs_bits(f[2][j]), abs_bits(f[3][j])));
        red[rq][cg * 8 + j] = am;
    }
    __syncthreads();
    if (t < kRhsCols) {
        uint32_t am = 0;
#pragma unroll 8
        for (int r = 0; r < 32; ++r) am = max(am, red[r][t]);
        const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
        mult[t] = g.m;
        if (n0 + t < N) s[kb * N + n0 + t] = g.s;
    }
    __syncthreads();
    uint32_t* tw = reinterpret_cast<uint32_t*>(tileT);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float mj = mult[cg * 8 + j];
        const uint32_t w = encode4_in_range<FNUZ>(f[0][j] * mj, f[1][j] * mj, f[2][j] * mj, f[3][j] * mj);
        const int cl = cg * 8 + j;
        const int chunk = (rq >> 2) ^ (cl >> 3);
        tw[cl * 32 + chunk * 4 + (rq & 3)] = w;
    }
    __syncthreads();
    // 8 consecutive lanes write one output row's 128 bytes: each store covers 8 whole lines
    const int chunk = t & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int cl = p * 32 + (t >> 3);
        const int64_t n = n0 + cl;
        if (n < N) {
            const uint4 v = tileT[cl * 8 + (chunk ^ (cl >> 3))];
            store16<VEC_Q>(qT + n * ldqT, k0 + chunk * 16, K, v);
        }
    }
}

// ------------------------------------------------------------------------------------------
// 128x1 of expert-grouped tokens: x [T, N] holds the tokens of E experts one after the other,
// expert e owning rows [offsets[e], offsets[e+1]) (clamped into [0, T] and to non-decreasing order).
// The 128x1 groups restart at every expert's first token, so an expert's last group may hold fewer
// than 128 tokens. The output puts expert e's tokens at padded position P[e] = the sum of the
// earlier experts' token counts, each rounded up to a multiple of 128: qT [N, *] holds at column
// P[e] + t the codes of the expert's token t and zeros in the columns up to the next multiple of
// 128; s holds the scale of padded group p (columns 128 p .. 128 p + 127) in row p. P (E + 1 values)
// is written too, for the grouped weight-gradient GEMM. A workgroup owns one padded group x 64
// columns, as in quantize_rhs_kernel; blockIdx.y runs over an upper bound of the padded groups
// (ceil(T / 128) + E) and the workgroups past the last group leave at once.
template <bool FNUZ, bool VEC_X, bool VEC_Q>
__global__ __launch_bounds__(256) void quantize_rhs_grouped_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t N, int64_t ldx, const int64_t* __restrict__ offsets,
    int64_t E, uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ s, int64_t* __restrict__ padded) {
    __shared__ uint32_t red[32][kRhsCols + 1];
    __shared__ float mult[kRhsCols];
    __shared__ uint4 tileT[kRhsCols * 8];

    const int t = threadIdx.x;
    const int cg = t & 7;
    const int rq = t >> 3;
    const int64_t gp = blockIdx.y;  // padded group
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRhsCols;
    const int64_t col = n0 + cg * 8;

    // this group's expert: scan the clamped boundaries (E is small); every workgroup of the first
    // group row writes P, each thread a part of it
    int64_t lo = 0, hi = 0, first = 0, prev = 0, groups_before = 0;
    bool found = false;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t a = min(max(offsets[e], prev), T);
        const int64_t b = min(max(offsets[e + 1], a), T);
        prev = b;
        const int64_t g = (b - a + kGroup - 1) / kGroup;
        if (!found && gp < groups_before + g) {
            found = true;
            lo = a;
            hi = b;
            first = groups_before;
        }
        if (blockIdx.x == 0 && gp == 0 && t == 0) padded[e] = groups_before * kGroup;
        groups_before += g;
    }
    if (blockIdx.x == 0 && gp == 0 && t == 0) padded[E] = groups_before * kGroup;
    if (!found) return;  // past the last padded group: the whole workgroup leaves

    const int64_t r0 = lo + (gp - first) * kGroup;  // the group's first token
    const int64_t rend = min(hi, r0 + kGroup);      // one past its last
    float f[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) load8<VEC_X>(x, ldx, r0 + rq * 4 + i, rend, col, N, f[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t am = max(max(abs_bits(f[0][j]), abs_bits(f[1][j])), max(abs_bits(f[2][j]), abs_bits(f[3][j])));
        red[rq][cg * 8 + j] = am;
    }
    __syncthreads();
    if (t < kRhsCols) {
        uint32_t am = 0;
#pragma unroll 8
        for (int r = 0; r < 32; ++r) am = max(am, red[r][t]);
        const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
        mult[t] = g.m;
        if (n0 + t < N) s[gp * N + n0 + t] = g.s;
    }
    __syncthreads();
    uint32_t* tw = reinterpret_cast<uint32_t*>(tileT);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float mj = mult[cg * 8 + j];
        const uint32_t w = encode4_in_range<FNUZ>(f[0][j] * mj, f[1][j] * mj, f[2][j] * mj, f[3][j] * mj);
        const int cl = cg * 8 + j;
        const int chunk = (rq >> 2) ^ (cl >> 3);
        tw[cl * 32 + chunk * 4 + (rq & 3)] = w;
    }
    __syncthreads();
    // the group's 128 padded columns of each output row (tokens past the expert's end are zeros)
    const int chunk = t & 7;
    const int64_t k0 = gp * kGroup;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int cl = p * 32 + (t >> 3);
        const int64_t n = n0 + cl;
        if (n < N) {
            const uint4 v = tileT[cl * 8 + (chunk ^ (cl >> 3))];
            store16<VEC_Q>(qT + n * ldqT, k0 + chunk * 16, k0 + kGroup, v);
        }
    }
}

// ------------------------------------------------------------------------------------------
// 128x128 blocks: one workgroup per block; thread t holds rows 8*(t/16) .. +8 x columns
// 8*(t%16) .. +8 (64 values in registers, read once). The block max is a wave reduction plus a
// 4-entry LDS combine. The optional transposed copy goes through a swizzled LDS tile.
template <bool FNUZ, bool VEC_W, bool VEC_Q, bool VEC_QT>
__global__ __launch_bounds__(256) void quantize_weight_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qT, int64_t ldqT,
    float* __restrict__ s, int64_t Kb) {
    __shared__ uint32_t wmax[4];
    __shared__ uint4 tileT[kGroup * 8];  // [column][8 x 16-byte chunks of rows], swizzled

    const int t = threadIdx.x;
    const int cg = t & 15;
    const int rg = t >> 4;
    const int64_t kb = blockIdx.x;
    const int64_t nb = blockIdx.y;
    const int64_t n0 = nb * kGroup;
    const int64_t k0 = kb * kGroup;
    const int64_t c = k0 + cg * 8;

    // the block stays packed as bf16 pairs (32 registers rather than 64 floats), so more
    // workgroups fit per CU
    uint32_t wv[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) load8_packed<VEC_W>(w, ldw, n0 + rg * 8 + i, N, c, K, wv[i]);
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) am = max(am, max((wv[i][d] << 16) & 0x7FFFFFFFu, wv[i][d] & 0x7FFF0000u));
    am = umax_wave(am);
    if ((t & 63) == 0) wmax[t >> 6] = am;
    __syncthreads();
    am = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
    if (t == 0) s[nb * Kb + kb] = g.s;

    uint32_t code[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        code[i][0] = encode4_in_range<FNUZ>(bf16_lo(wv[i][0]) * g.m, bf16_hi(wv[i][0]) * g.m,
                                            bf16_lo(wv[i][1]) * g.m, bf16_hi(wv[i][1]) * g.m);
        code[i][1] = encode4_in_range<FNUZ>(bf16_lo(wv[i][2]) * g.m, bf16_hi(wv[i][2]) * g.m,
                                            bf16_lo(wv[i][3]) * g.m, bf16_hi(wv[i][3]) * g.m);
        const int64_t n = n0 + rg * 8 + i;
        if (n < N) store8<VEC_Q>(q + n * ldq, c, K, code[i][0], code[i][1]);
    }
    if (qT == nullptr) return;  // uniform over the grid

    // 8x8 byte transpose: column j of my 8 columns collects byte j of rows 0..7.
    uint32_t* tw = reinterpret_cast<uint32_t*>(tileT);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int wsel = j >> 2;
        const int sh = 8 * (j & 3);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= ((code[i][wsel] >> sh) & 0xFFu) << (8 * i);
            hi |= ((code[i + 4][wsel] >> sh) & 0xFFu) << (8 * i);
        }
        const int cl = cg * 8 + j;
        const int chunk = (rg >> 1) ^ (cg & 7);
        const int idx = cl * 32 + chunk * 4 + (rg & 1) * 2;
        *reinterpret_cast<uint2*>(tw + idx) = make_uint2(lo, hi);
    }
    __syncthreads();
    // 8 consecutive lanes write one qT row's 128 bytes: each store covers 8 whole lines
    const int chunk = t & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int cl = p * 32 + (t >> 3);
        const int64_t k = k0 + cl;
        if (k < K) {
            const uint4 v = tileT[cl * 8 + (chunk ^ ((cl >> 3) & 7))];
            store16<VEC_QT>(qT + k * ldqT, n0 + chunk * 16, N, v);
        }
    }
}

// Value of lane l (0..7) of this lane's 16-lane DPP row (DPP row broadcast, control 0x150 + l);
// l is a constant once the caller's loop is unrolled.
__device__ __forceinline__ float bcast_row16(float v, int l) {
#define BSFP8_BC(L) \
    case L: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + L, 0xF, 0xF, false))
    switch (l) {
        BSFP8_BC(0); BSFP8_BC(1); BSFP8_BC(2); BSFP8_BC(3);
        BSFP8_BC(4); BSFP8_BC(5); BSFP8_BC(6); default: BSFP8_BC(7);
    }
#undef BSFP8_BC
}

// ------------------------------------------------------------------------------------------
// 1x128 and 128x1 of the same tensor in one pass: x [R, C] is read once and both the row-wise
// output of quantize_lhs (q [R, C], a_s column-major [R, ceil(C/128)]) and the transposed
// column-wise output of quantize_rhs (qT [C, R], s [ceil(R/128), C]) are written. A workgroup owns
// a 128 x 128 tile, which holds exactly one 1x128 group per row and one 128x1 group per column.
// Thread t holds rows 8 (t / 16) .. + 8 x columns 8 (t % 16) .. + 8; the 16 lanes of a DPP row
// share the rows, so a row maximum is one 16-lane DPP reduction; column maxima combine the 16 row
// groups through LDS. The transposed codes go through a swizzled LDS tile as in the weight kernel.
template <bool FNUZ, bool VEC_X, bool VEC_Q, bool VEC_QT>
__global__ __launch_bounds__(256, 4) void quantize_dual_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ a_s,
    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ s) {
    // the column-max scratch and the transposed code tile are never live together: one buffer
    // (16 KB + the 128 multipliers), so enough workgroups fit per CU for one wave of the grid
    __shared__ uint4 tileT[kGroup * 8];  // [column][8 x 16-byte chunks of rows], swizzled
    __shared__ float colm[kGroup];
    uint32_t (*red)[kGroup + 1] = reinterpret_cast<uint32_t (*)[kGroup + 1]>(tileT);
    static_assert(16 * (kGroup + 1) * 4 <= kGroup * 8 * 16, "column maxima fit in the tile buffer");

    const int t = threadIdx.x;
    const int cg = t & 15;
    const int rg = t >> 4;
    const int64_t cb = blockIdx.x;  // column block (K-block of the row-wise groups)
    const int64_t rb = blockIdx.y;  // row block (K-block of the column-wise groups)
    const int64_t r0 = rb * kGroup;
    const int64_t c0 = cb * kGroup;
    const int64_t c = c0 + cg * 8;

    // the tile stays packed as bf16 pairs (32 registers rather than 64 floats), so more waves fit
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        load8_packed<VEC_X>(x, ldx, r0 + rg * 8 + i, R, c, C, w[i]);
    }
    // element j (0..7) of row i as fp32, and its magnitude's bit pattern
    auto val = [&](int i, int j) { return (j & 1) ? bf16_hi(w[i][j >> 1]) : bf16_lo(w[i][j >> 1]); };
    auto mag = [&](int i, int j) {
        return (j & 1) ? (w[i][j >> 1] & 0x7FFF0000u) : ((w[i][j >> 1] << 16) & 0x7FFFFFFFu);
    };

    // column-wise partial maxima of this thread's 8 rows, combined over the 16 row groups in LDS
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = max(am, mag(i, j));
        red[rg][cg * 8 + j] = am;
    }

    // row-wise groups: max over the row's 128 columns (8 per lane x 16 lanes). Each of the 16 lanes
    // holds all 8 row maxima; lane cg computes the scale pair of row cg % 8 only, and every lane
    // then takes row i's pair from lane i of its DPP row (row broadcast).
    uint32_t rmax[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t am = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = max(am, mag(i, j));
        rmax[i] = umax_row16(am);
    }
    uint32_t mine = rmax[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mine = (cg & 7) == i ? rmax[i] : mine;
    const GroupScale gm = group_scale<FNUZ>(__uint_as_float(mine));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float m = bcast_row16(gm.m, i);
        const float sc = bcast_row16(gm.s, i);
        const uint32_t w0 = encode4_in_range<FNUZ>(val(i, 0) * m, val(i, 1) * m, val(i, 2) * m, val(i, 3) * m);
        const uint32_t w1 = encode4_in_range<FNUZ>(val(i, 4) * m, val(i, 5) * m, val(i, 6) * m, val(i, 7) * m);
        const int64_t r = r0 + rg * 8 + i;
        if (r < R) {  // rows >= R store neither codes nor scales
            store8<VEC_Q>(q + r * ldq, c, C, w0, w1);
            if (cg == 0) a_s[cb * R + r] = sc;
        }
    }

    // only the packed tile stays live across the barriers: the fp32 values are unpacked again below
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) asm volatile("" : "+v"(w[i][d]));
    __syncthreads();
    if (t < kGroup) {
        uint32_t am = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) am = max(am, red[r][t]);
        const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
        colm[t] = g.m;
        if (c0 + t < C) s[rb * C + c0 + t] = g.s;
    }
    __syncthreads();

    // column-wise codes, transposed through LDS: column j of my 8 collects byte j of rows 0..7
    uint32_t* tw = reinterpret_cast<uint32_t*>(tileT);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float mj = colm[cg * 8 + j];
        const uint32_t lo = encode4_in_range<FNUZ>(val(0, j) * mj, val(1, j) * mj, val(2, j) * mj, val(3, j) * mj);
        const uint32_t hi = encode4_in_range<FNUZ>(val(4, j) * mj, val(5, j) * mj, val(6, j) * mj, val(7, j) * mj);
        const int cl = cg * 8 + j;
        const int chunk = (rg >> 1) ^ (cg & 7);
        *reinterpret_cast<uint2*>(tw + cl * 32 + chunk * 4 + (rg & 1) * 2) = make_uint2(lo, hi);
    }
    __syncthreads();
    // 8 consecutive lanes write one column's 128 bytes, so each store instruction covers 8 whole
    // 128-byte lines of qT
    const int chunk = t & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int cl = p * 32 + (t >> 3);
        const int64_t col = c0 + cl;
        if (col < C) {
            const uint4 v = tileT[cl * 8 + (chunk ^ ((cl >> 3) & 7))];
            store16<VEC_QT>(qT + col * ldqT, r0 + chunk * 16, R, v);
        }
    }
}

// ------------------------------------------------------------------------------------------
// The two quantizations of a linear layer's forward step in one persistent launch: the 1x128
// row-wise groups of the activation x [M, K] (quantize_lhs) and the 128x128 blocks of the weight
// w [N, Kw] (quantize_weight_128x128, optional transposed copy). Both are cut into 128 x 128 tiles
// -- an activation tile holds one 1x128 group per row, a weight tile is one block -- and the
// resident workgroups (two per CU, 512 threads each) walk the joint tile list (activation tiles
// first). The workgroups of a CU drift apart, so one's loads overlap another's stores, and the two
// tensors share one ramp and one drain instead of paying two (4096 x 4096 each: 18.8 us against
// 21.7 us for the two kernels back to back). Thread t holds rows 4 (t / 16) .. + 4 x columns
// 8 (t % 16) .. + 8 of a tile as packed bf16 pairs (16 registers; with 256 threads and 8 rows
// each the kernel needed ~155 VGPRs and ran 4% slower at three workgroups per CU).
struct TileSrc {
    const uint16_t* base;
    int64_t ld, rows, cols, r0, c0;
};

constexpr int kStepThreads = 512;
constexpr int kStepRows = 4;        // rows per thread
constexpr int kStepWgPerCu = 2;

template <bool FNUZ, bool WANT_QT>
__global__ __launch_bounds__(kStepThreads, 1) void quantize_step_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ qx,
    int64_t ldqx, float* __restrict__ sx, const uint16_t* __restrict__ w, int64_t N, int64_t Kw,
    int64_t ldw, uint8_t* __restrict__ qw, int64_t ldqw, uint8_t* __restrict__ qwT, int64_t ldqwT,
    float* __restrict__ sw, int64_t kb_x, int64_t tiles_x, int64_t kb_w, int64_t tiles_w) {
    __shared__ uint4 tileT[kGroup * 8];  // transposed weight codes, [column][8 chunks], swizzled
    __shared__ uint32_t wmax[kStepThreads / 64];

    const int t = threadIdx.x;
    const int cg = t & 15;   // columns 8 cg .. 8 cg + 7 of the tile
    const int rg = t >> 4;   // rows 4 rg .. 4 rg + 3
    const int64_t total = tiles_x + tiles_w;

    for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
        TileSrc src;
        if (tile < tiles_x) {
            src = TileSrc{x, ldx, M, K, (tile / kb_x) * kGroup, (tile % kb_x) * kGroup};
        } else {
            const int64_t b = tile - tiles_x;
            src = TileSrc{w, ldw, N, Kw, (b / kb_w) * kGroup, (b % kb_w) * kGroup};
        }
        const int64_t c = src.c0 + cg * 8;
        uint32_t cur[kStepRows][4];
#pragma unroll
        for (int i = 0; i < kStepRows; ++i)
            load8_packed<true>(src.base, src.ld, src.r0 + rg * kStepRows + i, src.rows, c, src.cols, cur[i]);
        auto val = [&](int i, int j) { return (j & 1) ? bf16_hi(cur[i][j >> 1]) : bf16_lo(cur[i][j >> 1]); };
        auto mag = [&](int i, int j) {
            return (j & 1) ? (cur[i][j >> 1] & 0x7FFF0000u) : ((cur[i][j >> 1] << 16) & 0x7FFFFFFFu);
        };
        uint32_t code[kStepRows][2];
        if (tile < tiles_x) {
            // 1x128 groups: one per tile row; the row maximum is a 16-lane DPP reduction, lane
            // cg % 4 divides for row cg % 4 and every lane takes its rows' pairs by row broadcast
            uint32_t rmax[kStepRows];
#pragma unroll
            for (int i = 0; i < kStepRows; ++i) {
                uint32_t am = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) am = max(am, mag(i, j));
                rmax[i] = umax_row16(am);
            }
            uint32_t mine = rmax[0];
#pragma unroll
            for (int i = 1; i < kStepRows; ++i) mine = (cg & (kStepRows - 1)) == i ? rmax[i] : mine;
            const GroupScale gm = group_scale<FNUZ>(__uint_as_float(mine));
            const int64_t kb = src.c0 / kGroup;
            float sc[kStepRows];
#pragma unroll
            for (int i = 0; i < kStepRows; ++i) {
                const float m = bcast_row16(gm.m, i);
                sc[i] = bcast_row16(gm.s, i);
                code[i][0] = encode4_in_range<FNUZ>(val(i, 0) * m, val(i, 1) * m, val(i, 2) * m, val(i, 3) * m);
                code[i][1] = encode4_in_range<FNUZ>(val(i, 4) * m, val(i, 5) * m, val(i, 6) * m, val(i, 7) * m);
            }
#pragma unroll
            for (int i = 0; i < kStepRows; ++i) {
                const int64_t r = src.r0 + rg * kStepRows + i;
                if (r < M) {  // rows >= M store neither codes nor scales
                    store8<true>(qx + r * ldqx, c, K, code[i][0], code[i][1]);
                    if (cg == 0) sx[kb * M + r] = sc[i];
                }
            }
        } else {
            // one 128x128 block: wave maxima combined through LDS
            uint32_t am = 0;
#pragma unroll
            for (int i = 0; i < kStepRows; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) am = max(am, mag(i, j));
            am = umax_wave(am);
            if ((t & 63) == 0) wmax[t >> 6] = am;
            __syncthreads();
            am = wmax[0];
#pragma unroll
            for (int v = 1; v < kStepThreads / 64; ++v) am = max(am, wmax[v]);
            const GroupScale g = group_scale<FNUZ>(__uint_as_float(am));
            const int64_t nb = src.r0 / kGroup, kb = src.c0 / kGroup;
            if (t == 0) sw[nb * kb_w + kb] = g.s;
#pragma unroll
            for (int i = 0; i < kStepRows; ++i) {
                code[i][0] = encode4_in_range<FNUZ>(val(i, 0) * g.m, val(i, 1) * g.m, val(i, 2) * g.m, val(i, 3) * g.m);
                code[i][1] = encode4_in_range<FNUZ>(val(i, 4) * g.m, val(i, 5) * g.m, val(i, 6) * g.m, val(i, 7) * g.m);
            }
#pragma unroll
            for (int i = 0; i < kStepRows; ++i) {
                const int64_t n = src.r0 + rg * kStepRows + i;
                if (n < N) store8<true>(qw + n * ldqw, c, Kw, code[i][0], code[i][1]);
            }
            if (WANT_QT) {
                // column j of my 8 columns collects byte j of my 4 rows: one dword, rows 4 rg ..
                // 4 rg + 3 of column 8 cg + j, i.e. dword rg % 4 of 16-byte row chunk rg / 4; the
                // chunk is stored at position chunk ^ (column / 8) % 8
                uint32_t* tw = reinterpret_cast<uint32_t*>(tileT);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int wsel = j >> 2;
                    const int sh = 8 * (j & 3);
                    uint32_t d = 0;
#pragma unroll
                    for (int i = 0; i < kStepRows; ++i) d |= ((code[i][wsel] >> sh) & 0xFFu) << (8 * i);
                    const int cl = cg * 8 + j;
                    const int chunk = (rg >> 2) ^ (cg & 7);
                    tw[cl * 32 + chunk * 4 + (rg & 3)] = d;
                }
                __syncthreads();
                // 8 consecutive lanes write one qT row's 128 bytes
                const int chunk = t & 7;
#pragma unroll
                for (int p = 0; p < kGroup / (kStepThreads / 8); ++p) {
                    const int cl = p * (kStepThreads / 8) + (t >> 3);
                    const int64_t k = src.c0 + cl;
                    if (k < Kw) {
                        const uint4 v = tileT[cl * 8 + (chunk ^ ((cl >> 3) & 7))];
                        store16<true>(qwT + k * ldqwT, src.r0 + chunk * 16, N, v);
                    }
                }
            }
            __syncthreads();  // wmax and tileT are free for the next weight tile
        }
    }
}

// ------------------------------------------------------------------------------------------
// The element conversion on its own, for exhaustive checks: e4m3fn codes of arbitrary fp32 values
// (clamped to +-448), or the quantizers' float8_e4m3fnuz conversion (encode4_in_range<true> of
// twice the value) of values within the range a group multiplier produces.
template <bool FNUZ>
__device__ __forceinline__ uint32_t encode_one4(float a, float b, float c, float d) {
    return FNUZ ? encode4_in_range<true>(2.0f * a, 2.0f * b, 2.0f * c, 2.0f * d) : encode4(a, b, c, d);
}

template <bool FNUZ>
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ x,
                                                     uint8_t* __restrict__ q, int64_t n) {
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i0 + 4 <= n) {
        const float4 v = *reinterpret_cast<const float4*>(x + i0);
        const uint32_t w = encode_one4<FNUZ>(v.x, v.y, v.z, v.w);
        *reinterpret_cast<uint32_t*>(q + i0) = w;
    } else {
        for (int64_t i = i0; i < n; ++i)
            q[i] = static_cast<uint8_t>(encode_one4<FNUZ>(x[i], 0.f, 0.f, 0.f) & 0xFF);
    }
}

bool aligned(const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <bool FNUZ>
hipError_t quantize_lhs_impl(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                             int64_t ldq, float* a_s, int strip_loads, hipStream_t stream) {
    const int64_t Kb = (K + kGroup - 1) / kGroup;
    if (strip_loads >= 0 && aligned(x, 16) && ldx % 8 == 0 && aligned(q, 16) && ldq % 16 == 0 && K % 16 == 0) {
        const int nl = strip_loads > 0 ? strip_loads : sched::lhs_strip_loads(M, Kb, device_cus());
        const geom::StripShape sh = geom::strip_shape(M, Kb, nl);
        if (sh.units > 0x7FFFFFFFLL) return quantize_lhs_impl<FNUZ>(x, M, K, ldx, q, ldq, a_s, -1, stream);
        const dim3 grid(static_cast<unsigned>(sh.units));
#define BSFP8_QS(N) \
    quantize_lhs_strip_kernel<FNUZ, N><<<grid, geom::kStripThreads, 0, stream>>>(x, M, K, ldx, q, ldq, a_s, Kb, sh)
        switch (nl) {
            case 16: BSFP8_QS(16); break;
            case 8: BSFP8_QS(8); break;
            case 4: BSFP8_QS(4); break;
            case 2: BSFP8_QS(2); break;
            case 1: BSFP8_QS(1); break;
            default: return hipErrorInvalidValue;
        }
#undef BSFP8_QS
        return hipGetLastError();
    }
    const int64_t units = (M + kLhsRows - 1) / kLhsRows * Kb;
    const int64_t most = static_cast<int64_t>(device_cus()) * kLhsWgPerCu;
    const dim3 grid(static_cast<unsigned>(units < most ? units : most));
    const bool vx = aligned(x, 16) && (ldx % 8 == 0) && (K % 8 == 0);
    const bool vq = aligned(q, 8) && (ldq % 8 == 0) && (K % 8 == 0);
#define BSFP8_QL(A, B) \
    quantize_lhs_kernel<FNUZ, A, B><<<grid, 256, 0, stream>>>(x, M, K, ldx, q, ldq, a_s, Kb, units)
    if (vx && vq) BSFP8_QL(true, true);
    else if (vx) BSFP8_QL(true, false);
    else if (vq) BSFP8_QL(false, true);
    else BSFP8_QL(false, false);
#undef BSFP8_QL
    return hipGetLastError();
}

template <bool FNUZ>
hipError_t quantize_rhs_impl(const uint16_t* x, int64_t K, int64_t N, int64_t ldx, uint8_t* qT,
                             int64_t ldqT, float* s, hipStream_t stream) {
    const int64_t Kb = (K + kGroup - 1) / kGroup;
    const int64_t nc = (N + kRhsCols - 1) / kRhsCols;
    const int kb_fast = Kb * nc > static_cast<int64_t>(device_cus()) * kRhsWgPerCu && nc <= 65535;
    const dim3 grid = kb_fast ? dim3(static_cast<unsigned>(Kb), static_cast<unsigned>(nc))
                              : dim3(static_cast<unsigned>(nc), static_cast<unsigned>(Kb));
    const bool vx = aligned(x, 16) && (ldx % 8 == 0) && (N % 8 == 0);
    const bool vq = aligned(qT, 16) && (ldqT % 16 == 0) && (K % 16 == 0);
#define BSFP8_QR(A, B) \
    quantize_rhs_kernel<FNUZ, A, B><<<grid, 256, 0, stream>>>(x, K, N, ldx, qT, ldqT, s, kb_fast)
    if (vx && vq) BSFP8_QR(true, true);
    else if (vx) BSFP8_QR(true, false);
    else if (vq) BSFP8_QR(false, true);
    else BSFP8_QR(false, false);
#undef BSFP8_QR
    return hipGetLastError();
}

template <bool FNUZ>
hipError_t quantize_rhs_grouped_impl(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets,
                                     int64_t E, uint8_t* qT, int64_t ldqT, float* s, int64_t* padded,
                                     hipStream_t stream) {
    // at least the padded groups; one workgroup at least, which writes the padded offsets
    const int64_t groups = (T + kGroup - 1) / kGroup + E;
    const int64_t nc = (N + kRhsCols - 1) / kRhsCols;
    const dim3 grid(static_cast<unsigned>(nc > 0 ? nc : 1), static_cast<unsigned>(groups > 0 ? groups : 1));
    const bool vx = aligned(x, 16) && (ldx % 8 == 0) && (N % 8 == 0);
    const bool vq = aligned(qT, 16) && (ldqT % 16 == 0);
#define BSFP8_QG(A, B) \
    quantize_rhs_grouped_kernel<FNUZ, A, B><<<grid, 256, 0, stream>>>(x, T, N, ldx, offsets, E, qT, ldqT, s, padded)
    if (vx && vq) BSFP8_QG(true, true);
    else if (vx) BSFP8_QG(true, false);
    else if (vq) BSFP8_QG(false, true);
    else BSFP8_QG(false, false);
#undef BSFP8_QG
    return hipGetLastError();
}

template <bool FNUZ>
hipError_t quantize_weight_impl(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, uint8_t* qT, int64_t ldqT, float* s,
                                hipStream_t stream) {
    const int64_t Kb = (K + kGroup - 1) / kGroup;
    const int64_t Nb = (N + kGroup - 1) / kGroup;
    const dim3 grid(static_cast<unsigned>(Kb), static_cast<unsigned>(Nb));
    const bool vw = aligned(w, 16) && (ldw % 8 == 0) && (K % 8 == 0);
    const bool vq = aligned(q, 8) && (ldq % 8 == 0) && (K % 8 == 0);
    const bool vt = qT != nullptr && aligned(qT, 16) && (ldqT % 16 == 0) && (N % 16 == 0);
#define BSFP8_QW(A, B, C) \
    quantize_weight_kernel<FNUZ, A, B, C><<<grid, 256, 0, stream>>>(w, N, K, ldw, q, ldq, qT, ldqT, s, Kb)
    if (vw && vq && vt) BSFP8_QW(true, true, true);
    else if (vw && vq) BSFP8_QW(true, true, false);
    else if (vw && vt) BSFP8_QW(true, false, true);
    else if (vw) BSFP8_QW(true, false, false);
    else if (vq && vt) BSFP8_QW(false, true, true);
    else if (vq) BSFP8_QW(false, true, false);
    else if (vt) BSFP8_QW(false, false, true);
    else BSFP8_QW(false, false, false);
#undef BSFP8_QW
    return hipGetLastError();
}

template <bool FNUZ>
hipError_t quantize_dual_impl(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q,
                              int64_t ldq, float* a_s, uint8_t* qT, int64_t ldqT, float* s,
                              hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((C + kGroup - 1) / kGroup), static_cast<unsigned>((R + kGroup - 1) / kGroup));
    const bool vx = aligned(x, 16) && (ldx % 8 == 0) && (C % 8 == 0);
    const bool vq = aligned(q, 8) && (ldq % 8 == 0) && (C % 8 == 0);
    const bool vt = aligned(qT, 16) && (ldqT % 16 == 0) && (R % 16 == 0);
#define BSFP8_QD(A, B, D) \
    quantize_dual_kernel<FNUZ, A, B, D><<<grid, 256, 0, stream>>>(x, R, C, ldx, q, ldq, a_s, qT, ldqT, s)
    if (vx && vq && vt) BSFP8_QD(true, true, true);
    else if (vx && vq) BSFP8_QD(true, true, false);
    else if (vx && vt) BSFP8_QD(true, false, true);
    else if (vx) BSFP8_QD(true, false, false);
    else if (vq && vt) BSFP8_QD(false, true, true);
    else if (vq) BSFP8_QD(false, true, false);
    else if (vt) BSFP8_QD(false, false, true);
    else BSFP8_QD(false, false, false);
#undef BSFP8_QD
    return hipGetLastError();
}

template <bool FNUZ>
hipError_t quantize_step_impl(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qx,
                              int64_t ldqx, float* sx, const uint16_t* w, int64_t N, int64_t Kw,
                              int64_t ldw, uint8_t* qw, int64_t ldqw, uint8_t* qwT, int64_t ldqwT,
                              float* sw, hipStream_t stream) {
    const int64_t kb_x = (K + kGroup - 1) / kGroup, kb_w = (Kw + kGroup - 1) / kGroup;
    const int64_t tiles_x = (M + kGroup - 1) / kGroup * kb_x;
    const int64_t tiles_w = (N + kGroup - 1) / kGroup * kb_w;
    const int64_t want = static_cast<int64_t>(device_cus()) * kStepWgPerCu;
    const dim3 grid(static_cast<unsigned>(tiles_x + tiles_w < want ? tiles_x + tiles_w : want));
    if (qwT != nullptr)
        quantize_step_kernel<FNUZ, true><<<grid, kStepThreads, 0, stream>>>(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw,
                                                                   qwT, ldqwT, sw, kb_x, tiles_x, kb_w, tiles_w);
    else
        quantize_step_kernel<FNUZ, false><<<grid, kStepThreads, 0, stream>>>(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw,
                                                                    qwT, ldqwT, sw, kb_x, tiles_x, kb_w, tiles_w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_lhs(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                               int64_t ldq, float* a_s, bool fnuz, int strip_loads, hipStream_t stream) {
    return fnuz ? quantize_lhs_impl<true>(x, M, K, ldx, q, ldq, a_s, strip_loads, stream)
                : quantize_lhs_impl<false>(x, M, K, ldx, q, ldq, a_s, strip_loads, stream);
}

hipError_t launch_quantize_rhs(const uint16_t* x, int64_t K, int64_t N, int64_t ldx, uint8_t* qT,
                               int64_t ldqT, float* s, bool fnuz, hipStream_t stream) {
    return fnuz ? quantize_rhs_impl<true>(x, K, N, ldx, qT, ldqT, s, stream)
                : quantize_rhs_impl<false>(x, K, N, ldx, qT, ldqT, s, stream);
}

hipError_t launch_quantize_rhs_grouped(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets,
                                      int64_t E, uint8_t* qT, int64_t ldqT, float* s, int64_t* padded, bool fnuz,
                                      hipStream_t stream) {
    return fnuz ? quantize_rhs_grouped_impl<true>(x, T, N, ldx, offsets, E, qT, ldqT, s, padded, stream)
                : quantize_rhs_grouped_impl<false>(x, T, N, ldx, offsets, E, qT, ldqT, s, padded, stream);
}

hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                  int64_t ldq, uint8_t* qT, int64_t ldqT, float* s, bool fnuz,
                                  hipStream_t stream) {
    return fnuz ? quantize_weight_impl<true>(w, N, K, ldw, q, ldq, qT, ldqT, s, stream)
                : quantize_weight_impl<false>(w, N, K, ldw, q, ldq, qT, ldqT, s, stream);
}

hipError_t launch_quantize_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q,
                                int64_t ldq, float* a_s, uint8_t* qT, int64_t ldqT, float* s,
                                bool fnuz, hipStream_t stream) {
    return fnuz ? quantize_dual_impl<true>(x, R, C, ldx, q, ldq, a_s, qT, ldqT, s, stream)
                : quantize_dual_impl<false>(x, R, C, ldx, q, ldq, a_s, qT, ldqT, s, stream);
}

hipError_t launch_quantize_step(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qx,
                                int64_t ldqx, float* sx, const uint16_t* w, int64_t N, int64_t Kw,
                                int64_t ldw, uint8_t* qw, int64_t ldqw, uint8_t* qwT, int64_t ldqwT,
                                float* sw, bool fnuz, hipStream_t stream) {
    // the fused kernel takes the vector paths only: 16-byte bf16 rows with row lengths that are
    // multiples of 8, 8-byte code rows, 16-byte transposed rows; anything else runs the two
    // kernels one after the other
    const bool vec = aligned(x, 16) && ldx % 8 == 0 && K % 8 == 0 && aligned(w, 16) && ldw % 8 == 0 &&
                     Kw % 8 == 0 && aligned(qx, 8) &&
                     ldqx % 8 == 0 && aligned(qw, 8) && ldqw % 8 == 0 &&
                     (qwT == nullptr || (aligned(qwT, 16) && ldqwT % 16 == 0 && N % 16 == 0));
    if (!vec) {
        const hipError_t e = launch_quantize_lhs(x, M, K, ldx, qx, ldqx, sx, fnuz, 0, stream);
        if (e != hipSuccess) return e;
        return launch_quantize_weight(w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, fnuz, stream);
    }
    return fnuz ? quantize_step_impl<true>(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, stream)
                : quantize_step_impl<false>(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, stream);
}

hipError_t launch_encode(const float* x, uint8_t* q, int64_t n, bool fnuz, hipStream_t stream) {
    if (!aligned(x, 16) || !aligned(q, 4)) return hipErrorInvalidValue;
    const int64_t threads = (n + 3) / 4;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (fnuz)
        encode_kernel<true><<<grid, 256, 0, stream>>>(x, q, n);
    else
        encode_kernel<false><<<grid, 256, 0, stream>>>(x, q, n);
    return hipGetLastError();
}

}  // namespace bsfp8
