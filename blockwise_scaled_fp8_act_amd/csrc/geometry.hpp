// Index arithmetic of the gfx950 kernels: which rows, columns and scale elements each lane reads
// and writes, and the byte offsets it hands to the buffer loads. The kernels call these functions;
// tests/geometry_check.cpp compiles the same header for the CPU and enumerates every lane of every
// launch on ragged shapes, checking that each read is either inside its buffer or out of range as a
// whole, that every in-range element is read and written, and that nothing outside the tensors is
// written -- the checks "Mask a_s/b_s scale loads in blockwise FP8 training GEMM kernels" (Test)
// runs on its Triton kernels' offs_m / offs_n arithmetic, and the scale-store mask of the LHS
// quantizer from the root-cause comment of "Enable blockwise FP8 dense training kernels on ROCm".
//
// Buffer loads: a raw buffer resource of num_records bytes returns zero for an access whose
// per-lane offset (VGPR offset) lies at or past num_records (CDNA3/CDNA4 ISA, MUBUF out-of-range
// behaviour for raw buffers: stride 0, range checked on the byte offset). Every GEMM load here
// passes its whole offset in the VGPR (the scalar offset is always 0), every access is 16 bytes at a
// 16-byte-aligned offset into a buffer whose size is a multiple of 16, or 4 bytes at a 4-byte-aligned
// offset, so an access is entirely inside or entirely outside its buffer. A lane whose row, column
// or scale lies outside the tensor gets the offset kOob, to which only a per-K-block advance below
// 2^31 is added; the callers keep every buffer below kMaxRange bytes, so such an access is always
// out of range and never wraps past 2^32.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BSFP8_HD __host__ __device__ __forceinline__
#else
#define BSFP8_HD inline
#endif

namespace bsfp8 {
namespace geom {

constexpr uint32_t kOob = 0x80000000u;
constexpr int64_t kMaxRange = 0x80000000LL;  // buffer resources of the GEMMs span at most 2^31 bytes
constexpr int kBlockK = 128;                 // K-block depth (one 1x128 / 128x1 / 128x128 group)

// ---------------------------------------------------------------------------------------------
// Workgroup -> output tile (both GEMM kernels). Workgroups are dispatched round-robin over the 8
// XCDs; consecutive logical tiles go to one XCD, and logical tiles run in groups of kGroupRows
// tile-rows so the workgroups one XCD runs together share A rows and B columns in its L2.
constexpr int kXcds = 8;
constexpr int kGroupRows = 4;

BSFP8_HD void tile_of(int bid, int mt, int nt, int& tm, int& tn) {
    const int total = mt * nt;
    int logical = bid;
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    const int per_group = kGroupRows * nt;
    const int group = logical / per_group;
    const int first_m = group * kGroupRows;
    const int gsize = (mt - first_m) < kGroupRows ? (mt - first_m) : kGroupRows;
    const int in_group = logical - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// ---------------------------------------------------------------------------------------------
// Fast GEMM kernel: BM x 256 tiles of 2 BM / WM waves, BM = 256 with WM = 64 (8 waves) or BM = 128
// with WM = 64 (4 waves) or 32 (8 waves); wave w owns rows WM wm.. (wm = w % (BM / WM)) and columns
// 128 wn.. (wn = w / (BM / WM)) of the tile. Each K-block's operand tiles are loaded by the waves
// together, 16 bytes per lane, straight into LDS: every wave loads BM / waves rows of the A tile
// (32 or 16) and 256 / waves rows of the B tile (32 or 64).
constexpr int kFastBM = 256;
constexpr int kFastBN = 256;
constexpr int kFastBMSmall = 128;

// Operand load q (0 .. rows_per_wave / 8 - 1) of a wave whose share of the tile is rows_per_wave
// rows (32 for A; 32 or 64 for B): tile row rows_per_wave * wave + 8 q + lane / 8, 16-byte chunk
// (lane % 8) ^ swz(row) of the row's K-block, where swz(row) = (row / 2) % 8 is the LDS swizzle:
// lane l lands at LDS unit (rows_per_wave * wave + 8 q) * 8 + l = row * 8 + l % 8, which thus holds
// logical chunk (l % 8) ^ swz(row) (rows_per_wave * wave is a multiple of 32, so swz depends on q
// and l only). Load q reads through buffer resource q % 4, which starts at tile row 8 (q % 4) and
// spans the tile's in-range rows from there (fast_operand_range); the lane offset from that start,
// (rows_per_wave * wave + 32 (q / 4) + lane / 8) rows plus the chunk, depends on q only through
// q % 2 and q / 4, and a row past the matrix is past the end of the resource.
BSFP8_HD int fast_operand_row(int rows_per_wave, int wave, int q, int lane) {
    return rows_per_wave * wave + 8 * q + (lane >> 3);
}
BSFP8_HD int lds_swizzle(int row) { return (row >> 1) & 7; }
BSFP8_HD int fast_operand_chunk(int q, int lane) { return (lane & 7) ^ ((4 * (q & 1) + (lane >> 4)) & 7); }
// Per-lane offset of load q from the start of its resource, before the K-block advance kb * 128.
BSFP8_HD uint32_t fast_operand_lane(int rows_per_wave, int wave, int q, int lane, int64_t ld) {
    return static_cast<uint32_t>((rows_per_wave * wave + 32 * (q >> 2) + (lane >> 3)) * ld +
                                 16 * fast_operand_chunk(q, lane));
}
// Resource of load q: from tile row 8 (q % 4), (rows_in_range - 8 (q % 4)) rows of ld bytes (none
// if negative).
BSFP8_HD int64_t fast_operand_first_row(int q) { return 8 * (q & 3); }
BSFP8_HD int64_t fast_operand_range(int q, int64_t rows_in_range, int64_t ld) {
    return rows_in_range > 8 * (q & 3) ? (rows_in_range - 8 * (q & 3)) * ld : 0;
}
BSFP8_HD uint32_t fast_operand_advance(int64_t kb) { return static_cast<uint32_t>(kb * kBlockK); }

// A scales of a K-block: lanes 0 .. rows_per_wave - 1 of each wave (rows_per_wave = the A rows a
// wave loads, 32 or 16) load one fp32 each, tile row rows_per_wave wave + lane (LDS float of the
// same index). a_s is column-major [M, Kb] with ld M: element (m, kb) at kb * M + m.
BSFP8_HD uint32_t fast_ascale_base(int rows_per_wave, int64_t m0, int64_t m_end, int wave, int lane) {
    const int64_t m = m0 + rows_per_wave * wave + lane;
    return (lane < rows_per_wave && m < m_end) ? static_cast<uint32_t>(4 * m) : kOob;
}
BSFP8_HD uint32_t fast_ascale_advance(int64_t kb, int64_t M) { return static_cast<uint32_t>(4 * kb * M); }

// Per-column B scales of a K-block: lanes 0 .. cols_per_wave - 1 of each wave (cols_per_wave =
// 256 / waves: 32 or 64), tile column cols_per_wave * wave + lane (LDS float of the same index);
// b_s [Kb, N] row-major: element (kb, n) at kb * N + n.
BSFP8_HD uint32_t fast_bscale_col_base(int cols_per_wave, int64_t n0, int64_t N, int wave, int lane) {
    const int64_t n = n0 + cols_per_wave * wave + lane;
    return (lane < cols_per_wave && n < N) ? static_cast<uint32_t>(4 * n) : kOob;
}
BSFP8_HD uint32_t fast_bscale_col_advance(int64_t kb, int64_t N) { return static_cast<uint32_t>(4 * kb * N); }

// 128x128 B scales of a K-block: lanes 0 and 1 of wave 0, column block 2 tn + lane (LDS float lane);
// element (kb, nb) at nb * bs_nb + kb * bs_kb.
BSFP8_HD uint32_t fast_bscale_blk_base(int tn, int64_t N, int64_t bs_nb, int wave, int lane) {
    const int64_t nb = 2 * static_cast<int64_t>(tn) + lane;
    return (wave == 0 && lane < 2 && nb * kBlockK < N) ? static_cast<uint32_t>(4 * nb * bs_nb) : kOob;
}
BSFP8_HD uint32_t fast_bscale_blk_advance(int64_t kb, int64_t bs_kb) { return static_cast<uint32_t>(4 * kb * bs_kb); }
// floats a strided 128x128 scale tensor spans: the largest index read plus one
BSFP8_HD int64_t bscale_blk_extent(int64_t N, int64_t Kb, int64_t bs_nb, int64_t bs_kb) {
    const int64_t Nb = (N + kBlockK - 1) / kBlockK;
    return (Nb - 1) * bs_nb + (Kb - 1) * bs_kb + 1;
}

// Bytes of the last K-block that lie below K and the fragment mask: register d of lane group lg
// holds row bytes from 16 lg + 4 d (d < 4) and from 64 + 16 lg + 4 (d - 4) (d >= 4) in both
// operands; bytes at and past krem are zeroed.
BSFP8_HD int fragment_byte(int lg, int d) { return d < 4 ? 16 * lg + 4 * d : 64 + 16 * lg + 4 * (d - 4); }
BSFP8_HD uint32_t tail_keep_mask(int krem, int lg, int d) {
    const int keep = krem - fragment_byte(lg, d);
    return keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
}

// bf16 epilogue: pass p (0 .. WM / 4 - 1) of a wave (a block of WM = 64 or 32 rows) stores 16 bytes
// per lane: row WM wm + 4 p + lane / 16, columns 128 wn + 8 (lane % 16) .. + 8 of the tile; element
// n + e is stored iff row < m_end and n + e < N.
BSFP8_HD int64_t fast_store_row(int wave_rows, int64_t m0, int wm, int p, int lane) {
    return m0 + wave_rows * wm + 4 * p + (lane >> 4);
}
BSFP8_HD int64_t fast_store_col(int64_t n0, int wn, int lane) { return n0 + 128 * wn + 8 * (lane & 15); }

// fp32 partial epilogue (split K): subtile (i, j) of a wave stores a lane's four totals at row
// WM wm + 16 i + lane % 16, columns 128 wn + 16 j + 4 (lane / 16) .. + 4 of the tile, iff the row is
// below m_end and the first column below N (the partial rows are padded to a multiple of 4 floats).
BSFP8_HD int64_t fast_partial_row(int wave_rows, int64_t m0, int wm, int i, int lane) {
    return m0 + wave_rows * wm + 16 * i + (lane & 15);
}
BSFP8_HD int64_t fast_partial_col(int64_t n0, int wn, int j, int lane) { return n0 + 128 * wn + 16 * j + 4 * (lane >> 4); }

// Split K: slice s of S owns K-blocks [split_begin(Kb, S, s), split_begin(Kb, S, s + 1)).
BSFP8_HD int64_t split_begin(int64_t Kb, int64_t S, int64_t s) { return Kb * s / S; }

// ---------------------------------------------------------------------------------------------
// Thin GEMM kernel (problems with few rows): 64 x bn tiles, bn = 32, 64 or 128, 4 waves; wave w owns
// rows 32 (w % 2).. and columns (bn / 2) (w / 2).. of the tile. A K-block's tile is (64 + bn) rows
// of 128 bytes (A rows 0..63, then B rows 0..bn-1), loaded in groups of 8 rows, one 16-byte chunk
// per lane; the 8 + bn / 8 groups are dealt to the waves in order, thin_loads(bn) each. Each operand
// is read through one resource that starts at the tile's first row and spans its in-range rows, so
// a row past M or N is past the end of the resource.
constexpr int kThinBM = 64;
// A thin workgroup has 4 waves (2 x 2, each 32 x bn/2) or, for bn >= 64, 8 (4 x 2, each 16 x bn/2).
BSFP8_HD int thin_rows_per_wave(int waves) { return 2 * kThinBM / waves; }
BSFP8_HD int thin_loads(int bn, int waves) { return (kThinBM + bn) / (8 * waves); }
// LDS image of one pipeline stage, in 16-byte units: A rows 0..63 and B rows 0..bn-1 (8 units of
// 128 bytes each), the 64 A scales, then the B scales (per column: bn floats; 128x128: one float).
constexpr int thin_stage_units(int bn, bool per_col) { return (kThinBM + bn) * 8 + kThinBM / 4 + (per_col ? bn / 4 : 1); }
// The thin kernel's LDS pipeline of `stages` stages: K-block b lives in stage b % stages; one
// iteration waits for its n blocks (n = thin_blocks_per_step, or 1 for the last few), passes one
// barrier, issues the n blocks thin_ahead blocks after its first, and multiplies its blocks; the
// prologue issues blocks 0 .. thin_ahead - 1.
BSFP8_HD constexpr int thin_blocks_per_step(int stages) { return stages >= 12 ? 4 : stages >= 4 ? 2 : 1; }
BSFP8_HD constexpr int thin_ahead(int stages) { return stages - thin_blocks_per_step(stages); }
BSFP8_HD constexpr int thin_stage_of(int stages, int kb) { return kb % stages; }
// Blocks that may still be in flight when the iteration for blocks kb .. kb + n - 1 (of Kb) waits.
BSFP8_HD int thin_wait_later(int stages, int kb, int n, int Kb) {
    const int a = thin_ahead(stages) - n, b = Kb - kb - n;
    return a < b ? a : b;
}
// Load p (0 .. thin_loads(bn, waves) - 1) of wave w: row group g = w thin_loads + p of the tile; A's
// groups are 0..7, B's follow. thin_group: the group's index within its operand.
BSFP8_HD bool thin_load_is_a(int bn, int waves, int wave, int p) { return wave * thin_loads(bn, waves) + p < kThinBM / 8; }
BSFP8_HD int thin_group(int bn, int waves, int wave, int p) {
    const int g = wave * thin_loads(bn, waves) + p;
    return g < kThinBM / 8 ? g : g - kThinBM / 8;
}
// Lane l of a load of group gr: operand row 8 gr + l / 8, chunk (l % 8) ^ swz(row) (the LDS swizzle
// of the fast kernel, lds_swizzle), landing at LDS unit (operand base) + 64 gr + l = row 8 + l % 8.
BSFP8_HD int thin_operand_row(int gr, int lane) { return 8 * gr + (lane >> 3); }
BSFP8_HD uint32_t thin_operand_lane(int gr, int lane, int64_t ld) {
    return static_cast<uint32_t>(thin_operand_row(gr, lane) * ld + 16 * fast_operand_chunk(gr, lane));
}
BSFP8_HD int64_t thin_operand_range(int64_t rows_in_range, int64_t ld) { return rows_in_range > 0 ? rows_in_range * ld : 0; }
// LDS unit (16 bytes) of lane 0 of the load, within a stage: A rows at 0, B rows at 64 * 8.
BSFP8_HD int thin_load_unit(int bn, int waves, int wave, int p) {
    return (thin_load_is_a(bn, waves, wave, p) ? 0 : kThinBM * 8) + 64 * thin_group(bn, waves, wave, p);
}
// Scale loads of a K-block: wave 0 loads the A scales of the tile's 64 rows (lane = tile row, LDS
// float lane); the B scales come from wave 3 (per column: tile columns 0..63, LDS float = column;
// 128x128: lane 0 alone, the scale of the tile's 128-column block) and, for the per-column scales
// of a 128-column tile, from wave 2 (columns 64..127).
BSFP8_HD uint32_t thin_ascale_base(int64_t m0, int64_t M, int lane) {
    return m0 + lane < M ? static_cast<uint32_t>(4 * (m0 + lane)) : kOob;
}
BSFP8_HD bool thin_has_bscale_load(int bn, bool per_col, int wave) { return wave == 3 || (per_col && bn > 64 && wave == 2); }
BSFP8_HD int thin_bscale_col(int wave, int lane) { return (wave == 2 ? 64 : 0) + lane; }
BSFP8_HD uint32_t thin_bscale_col_base(int bn, int64_t n0, int64_t N, int wave, int lane) {
    const int c = thin_bscale_col(wave, lane);
    return (lane < bn && c < bn && n0 + c < N) ? static_cast<uint32_t>(4 * (n0 + c)) : kOob;
}
// Lanes switched on for a B-scale load (a direct load writes LDS for every active lane, in range or
// not): per column, lanes 0 .. bn - 1 (at most 64); 128x128, lane 0.
BSFP8_HD uint64_t thin_bscale_lanes(int bn, bool per_col) {
    return !per_col ? 1ull : (bn >= 64 ? ~0ull : ((1ull << bn) - 1));
}
BSFP8_HD uint32_t thin_bscale_blk_base(int64_t n0, int64_t bs_nb, int lane) {
    return lane == 0 ? static_cast<uint32_t>(4 * (n0 / kBlockK) * bs_nb) : kOob;
}
// Output of subtile (i, j) of wave (wm, wn) (wm = wave % (waves / 2), wn = wave / (waves / 2)): row
// thin_rows_per_wave wm + 16 i + lane % 16 and columns (bn / 2) wn + 16 j + 4 (lane / 16) .. + 4
// of the tile; element n + e is stored iff the row is below M and n + e < N.
BSFP8_HD int64_t thin_store_row(int64_t m0, int waves, int wm, int i, int lane) {
    return m0 + thin_rows_per_wave(waves) * wm + 16 * i + (lane & 15);
}
BSFP8_HD int64_t thin_store_col(int64_t n0, int bn, int wn, int j, int lane) {
    return n0 + (bn / 2) * wn + 16 * j + 4 * (lane >> 4);
}

// ---------------------------------------------------------------------------------------------
// General GEMM kernel (float8_e4m3fnuz operands): 256 x 128 tile, 8 waves (wm = wave / 2 owns rows
// 64 wm.., wn = wave % 2 columns 64 wn..), operands read through buffer loads into registers.
constexpr int kGenBM = 256;
constexpr int kGenBN = 128;

// A fragment of subtile i (0..3): tile row 64 wm + 16 i + lane % 16, bytes [32 (lane / 16), +32)
// of the K-block as two 16-byte loads (the second at +16). Subtile i reads through its own resource
// from tile row 16 i (gen_a_range), so the lane offset is the same for every i.
BSFP8_HD int gen_a_row(int wm, int i, int lane) { return 64 * wm + 16 * i + (lane & 15); }
BSFP8_HD int64_t gen_a_first_row(int i) { return 16 * i; }
BSFP8_HD int64_t gen_a_range(int i, int64_t rows_in_range, int64_t lda) {
    return rows_in_range > 16 * i ? (rows_in_range - 16 * i) * lda : 0;
}
BSFP8_HD uint32_t gen_a_lane(int wm, int lane, int64_t lda) {
    return static_cast<uint32_t>((64 * wm + (lane & 15)) * lda + 32 * (lane >> 4));
}
// B tile rows into registers (a partial last K-block): thread t (0..511) loads row t / 8 + 64 p
// (p = 0, 1), 16-byte chunk t % 8, through the resource from tile row 64 p; LDS row r holds chunk c
// at position c ^ (r % 8).
BSFP8_HD int gen_b_row(int tid, int p) { return (tid >> 3) + 64 * p; }
BSFP8_HD int64_t gen_b_first_row(int p) { return 64 * p; }
BSFP8_HD int64_t gen_b_range(int p, int64_t rows_in_range, int64_t ldb) {
    return rows_in_range > 64 * p ? (rows_in_range - 64 * p) * ldb : 0;
}
BSFP8_HD uint32_t gen_b_lane(int tid, int64_t ldb) { return static_cast<uint32_t>((tid >> 3) * ldb + 16 * (tid & 7)); }
// B tile of a full K-block straight into LDS: load q (0, 1) of wave w, lane l: row 16 w + 8 q + l / 8,
// LDS position l % 8 holding logical chunk (l % 8) ^ (row % 8) = (l % 8) ^ (l / 8), through the
// resource from tile row 8 q.
BSFP8_HD int gen_bdma_row(int wave, int q, int lane) { return 16 * wave + 8 * q + (lane >> 3); }
BSFP8_HD int64_t gen_bdma_first_row(int q) { return 8 * q; }
BSFP8_HD int64_t gen_bdma_range(int q, int64_t rows_in_range, int64_t ldb) {
    return rows_in_range > 8 * q ? (rows_in_range - 8 * q) * ldb : 0;
}
BSFP8_HD uint32_t gen_bdma_lane(int wave, int lane, int64_t ldb) {
    return static_cast<uint32_t>((16 * wave + (lane >> 3)) * ldb + 16 * ((lane & 7) ^ (lane >> 3)));
}
// A scale of subtile i's row (element (m, kb) of the column-major a_s at 4 (kb M + m)): the lane's
// base, kOob for a row >= M; the K-block advance 4 kb M is added per load.
BSFP8_HD uint32_t gen_ascale_base(int64_t m0, int wm, int i, int lane, int64_t M) {
    const int64_t m = m0 + gen_a_row(wm, i, lane);
    return m < M ? static_cast<uint32_t>(4 * m) : kOob;
}
// Output columns n .. n + 3 of subtile j: n = n0 + 64 wn + 16 j + 4 (lane / 16).
BSFP8_HD int64_t gen_col(int64_t n0, int wn, int j, int lane) { return n0 + 64 * wn + 16 * j + 4 * (lane >> 4); }
// Per-column B scales of a K-block, staged in LDS: thread tid < 128 loads the scale of tile column
// tid (LDS float tid), base 4 (n0 + tid), kOob for the other threads and for columns >= N; advance
// 4 kb N.
BSFP8_HD uint32_t gen_bscale_tile_base(int64_t n0, int64_t N, int tid) {
    return (tid < kGenBN && n0 + tid < N) ? static_cast<uint32_t>(4 * (n0 + tid)) : kOob;
}

// ---------------------------------------------------------------------------------------------
// Quantizer scale stores. Each function gives the scale element a thread writes and whether it
// writes it; the kernels store exactly when the predicate holds.

// quantize_lhs: unit u (kLhsRows rows of one K-block, K-block fastest) of a 256-thread workgroup;
// team = thread / 16 (16 teams), r = 0..rows_per_team-1: row rb * 16 * rows_per_team + 16 r + team;
// lane 0 of each team stores a_s[kb * M + row] iff row < M.
BSFP8_HD void lhs_unit(int64_t u, int64_t Kb, int64_t& rb, int64_t& kb) {
    rb = u / Kb;
    kb = u - rb * Kb;
}
BSFP8_HD int64_t lhs_row(int64_t rb, int rows_per_team, int r, int team) {
    return rb * 16 * rows_per_team + 16 * r + team;
}
BSFP8_HD int64_t colmajor_index(int64_t kb, int64_t M, int64_t m) { return kb * M + m; }
// a row's codes and scale are stored only when the row is inside the tensor
BSFP8_HD bool row_stored(int64_t m, int64_t M) { return m < M; }

// quantize_lhs, row strips (the path for K % 16 == 0 with 16-byte aligned rows). A 512-thread
// workgroup owns a strip: `rows` consecutive rows times a chunk of g K-blocks. Its bf16 input is
// cut into 16-byte pieces numbered row-major, p = r * 16 g + cp (cp: the 8-column piece of the
// chunk row); thread t loads pieces t + 512 j. A 1x128 group is 16 aligned consecutive pieces, so
// its 16 lanes are one aligned 16-lane row of a wave. The codes go to LDS row-major and leave as
// 16-byte pieces numbered the same way, s = r * 8 g + cs; the chunk's scales leave K-block by
// K-block, `rows` consecutive floats of a column-major scale column each.
constexpr int kStripThreads = 512;
struct StripShape {
    int rows;        // rows per strip
    int g;           // K-blocks per chunk
    int loads;       // 16-byte input pieces per thread (the last may be partial across the workgroup)
    int64_t chunks;  // chunks per row
    int64_t units;   // workgroups: strips x chunks, chunk fastest
};
// Strip of `loads_max` pieces per thread: chunks of at most 32 K-blocks split K evenly, and as many
// rows as fill 512 x loads_max pieces.
BSFP8_HD StripShape strip_shape(int64_t M, int64_t Kb, int loads_max) {
    StripShape s;
    s.chunks = (Kb + 31) / 32;
    s.g = static_cast<int>((Kb + s.chunks - 1) / s.chunks);
    s.rows = kStripThreads * loads_max / (16 * s.g);
    s.loads = (s.rows * 16 * s.g + kStripThreads - 1) / kStripThreads;
    s.units = (M + s.rows - 1) / s.rows * s.chunks;
    return s;
}
BSFP8_HD void strip_unit(int64_t u, int64_t chunks, int64_t& strip, int64_t& chunk) {
    strip = u / chunks;
    chunk = u - strip * chunks;
}
// input piece p of the strip: row m0 + p / (16 g), columns c0 + 8 (p % (16 g)) .. + 7; it holds
// data when p < rows * 16 g, the row is < M and the column < K (K % 8 == 0: all 8 or none)
BSFP8_HD bool strip_piece(int p, const StripShape& s, int64_t m0, int64_t c0, int64_t M, int64_t K,
                          int64_t& m, int64_t& c) {
    const int per_row = 16 * s.g;
    m = m0 + p / per_row;
    c = c0 + 8 * (p % per_row);
    return p < s.rows * per_row && m < M && c < K;
}
// output piece q of the strip (16 code bytes): row m0 + q / (8 g), byte column c0 + 16 (q % (8 g));
// stored when q < rows * 8 g, the row is < M and the column < K (K % 16 == 0: all 16 or none)
BSFP8_HD bool strip_out_piece(int q, const StripShape& s, int64_t m0, int64_t c0, int64_t M, int64_t K,
                              int64_t& m, int64_t& c) {
    const int per_row = 8 * s.g;
    m = m0 + q / per_row;
    c = c0 + 16 * (q % per_row);
    return q < s.rows * per_row && m < M && c < K;
}
// scale i of the strip (i < rows * g): K-block kb0 + i / rows of row m0 + i % rows, stored at
// a_s[kb * M + m] when the row is < M and the K-block < Kb
BSFP8_HD bool strip_scale(int i, const StripShape& s, int64_t m0, int64_t kb0, int64_t M, int64_t Kb,
                          int64_t& kb, int64_t& m) {
    kb = kb0 + i / s.rows;
    m = m0 + i % s.rows;
    return i < s.rows * s.g && m < M && kb < Kb;
}

}  // namespace geom
}  // namespace bsfp8
