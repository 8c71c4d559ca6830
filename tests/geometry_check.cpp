// Host-side check of the GEMM kernels' index arithmetic (blockwise_scaled_fp8_act_amd/csrc/
// geometry.hpp, the same header the kernels call), in the manner of the index test of "Mask a_s/b_s
// scale loads in blockwise FP8 training GEMM kernels" (Test): for ragged M, N, K it enumerates every
// lane of every workgroup and K-block and asserts
//   * every buffer access is 16-byte (operands) or 4-byte (scales) aligned and lies wholly inside or
//     wholly outside its buffer resource, offsets never wrap past 2^32, and an access inside its
//     resource is inside the tensor it was built over;
//   * a lane whose row / column / scale is outside the tensor is outside its resource (it reads zero);
//   * every in-range operand chunk and scale is loaded exactly once per K-block, into the LDS slot
//     the fragment reads expect;
//   * every output element (m < M, n < N) is stored exactly once and nothing else is stored (bf16
//     epilogue, split-K partial tiles), and the split slices partition the K-blocks;
//   * the partial-K-block masks keep exactly the fragment bytes below K;
//   * quantize_lhs stores each scale of the column-major [M, Kb] tensor exactly once and never a row
//     >= M (the root-cause comment of "Enable blockwise FP8 dense training kernels on ROCm"), in its
//     tile kernel and in its row-strip kernel (whose code reads and stores are checked too).
// The fast kernel's three tile shapes (256 rows, 8 waves of 64 rows; 128 rows, 4 waves of 64 rows or
// 8 waves of 32 rows) and the thin kernel's tiles (64 rows by 32, 64 or 128 columns in 4 waves;
// 64 or 128 columns in 8 waves) are enumerated.
// Usage: geometry_check M N K [M N K ...]; prints one line per shape, exits 1 on the first failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

#include "geometry.hpp"

using namespace bsfp8::geom;

static int g_fail = 0;
#define CHECK(cond, ...)                                              \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
            std::printf(__VA_ARGS__);                                 \
            std::printf("\n");                                        \
            g_fail = 1;                                               \
            return false;                                             \
        }                                                             \
    } while (0)

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One access of `size` bytes at 64-bit offset `off` (the value the lane hands the hardware, reduced
// to 32 bits) into a resource of `range` bytes: returns true if it reads memory (in range).
static bool access(uint64_t off, int64_t range, int size, bool& ok) {
    ok = off < (1ull << 32) && off % size == 0 && range % size == 0;
    return static_cast<int64_t>(off) < range;
}

// ---------------------------------------------------------------------------------------------
static bool check_tiles(int mt, int nt) {
    std::vector<int> seen(static_cast<size_t>(mt) * nt, 0);
    for (int bid = 0; bid < mt * nt; ++bid) {
        int tm, tn;
        tile_of(bid, mt, nt, tm, tn);
        CHECK(tm >= 0 && tm < mt && tn >= 0 && tn < nt, "bid %d -> (%d, %d) of %d x %d", bid, tm, tn, mt, nt);
        CHECK(++seen[static_cast<size_t>(tm) * nt + tn] == 1, "tile (%d, %d) twice", tm, tn);
    }
    return true;
}

// Fast kernel operand loads of one tile and K-block: rows [0, rows) of a tile starting at row r0 of an
// operand with `total_rows` rows of K bytes at row stride ld. A chunk that holds bytes below K must be
// read at its address; a chunk wholly at or past K (masked to zero in the fragments) may read the
// following bytes of the operand or nothing, but never outside it.
// rpw: rows each of the `waves` waves loads (8 per load instruction).
static bool check_fast_operand(int64_t r0, int64_t rows, int64_t total_rows, int64_t ld, int64_t K, int64_t kb,
                               int rpw, int waves) {
    std::vector<uint8_t> got(static_cast<size_t>(rpw) * waves * 8, 0);
    for (int q = 0; q < rpw / 8; ++q) {
        const int64_t range = fast_operand_range(q, rows, ld);
        const int64_t first = r0 + fast_operand_first_row(q);
        for (int wave = 0; wave < waves; ++wave)
            for (int lane = 0; lane < 64; ++lane) {
                const uint64_t off = static_cast<uint64_t>(fast_operand_lane(rpw, wave, q, lane, ld)) + fast_operand_advance(kb);
                bool ok;
                const bool in = access(off, range, 16, ok);
                CHECK(ok, "operand offset %llu (range %lld)", (unsigned long long)off, (long long)range);
                const int r = fast_operand_row(rpw, wave, q, lane);
                const int c = fast_operand_chunk(q, lane);
                // LDS slot of the lane: unit (rpw wave + 8 q) * 8 + lane = row r, position lane % 8,
                // which the fragment reads take as logical chunk (lane % 8) ^ swizzle(r)
                CHECK((rpw * wave + 8 * q) * 8 + lane == r * 8 + (lane & 7), "LDS unit");
                CHECK(((lane & 7) ^ lds_swizzle(r)) == c, "LDS chunk position");
                const bool needed = kb * kBlockK + 16 * c < K;
                if (r < rows) {
                    CHECK(static_cast<int64_t>(off) == (r - fast_operand_first_row(q)) * ld + kb * kBlockK + 16 * c, "operand address");
                    if (needed) {
                        CHECK(in, "row %d chunk %d below K not read (q %d wave %d lane %d)", r, c, q, wave, lane);
                        CHECK(++got[r * 8 + c] == 1, "row %d chunk %d loaded twice", r, c);
                    }
                } else {
                    CHECK(!in, "row %d past the tile's %lld rows is read", r, (long long)rows);
                }
                if (in) CHECK(first * ld + static_cast<int64_t>(off) + 16 <= total_rows * ld, "read past the operand");
            }
    }
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < 8; ++c)
            if (kb * kBlockK + 16 * c < K) CHECK(got[r * 8 + c] == 1, "row %d chunk %d not loaded", r, c);
    return true;
}

// bm: the tile height; wr: the rows of a wave's block (256 / 64: 8 waves; 128 / 64: 4 waves; 128 /
// 32: 8 waves). Each wave loads bm / waves rows of A and 256 / waves rows of B.
static bool check_fast(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int bm, int wr) {
    const int wms = bm / wr, waves = 2 * wms, cpw = kFastBN / waves, apw = bm / waves;
    const int mt = static_cast<int>(cdiv(M, bm)), nt = static_cast<int>(cdiv(N, kFastBN));
    const int64_t Kb = cdiv(K, kBlockK);
    if (!check_tiles(mt, nt)) return false;
    // 128x128 B scales read with the forward strides (Kb, 1) and the dgrad strides (1, Nb)
    const int64_t Nb = cdiv(N, kBlockK);
    const int64_t strides[2][2] = {{Kb, 1}, {1, Nb}};
    std::vector<uint8_t> stored(static_cast<size_t>(M) * N, 0);
    for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < nt; ++tn) {
            const int64_t m0 = static_cast<int64_t>(tm) * bm, n0 = static_cast<int64_t>(tn) * kFastBN;
            const int64_t arows = M - m0 < bm ? M - m0 : bm;
            const int64_t brows = N - n0 < kFastBN ? N - n0 : kFastBN;
            for (int64_t kb = 0; kb < Kb; ++kb) {
                if (!check_fast_operand(m0, arows, M, lda, K, kb, apw, waves)) return false;
                if (!check_fast_operand(n0, brows, N, ldb, K, kb, cpw, waves)) return false;
                // A scales: lanes 0 .. apw - 1 of each wave (the others are switched off); per-column
                // B scales: lanes 0 .. cpw - 1
                std::vector<uint8_t> sa(256, 0), sbc(256, 0);
                for (int wave = 0; wave < waves; ++wave)
                    for (int lane = 0; lane < 64; ++lane) {
                        bool ok;
                        if (lane < apw) {
                            const uint64_t off = static_cast<uint64_t>(fast_ascale_base(apw, m0, M, wave, lane)) + fast_ascale_advance(kb, M);
                            const bool in = access(off, 4 * M * Kb, 4, ok);
                            CHECK(ok, "a_s offset");
                            const int64_t m = m0 + apw * wave + lane;
                            CHECK(apw * wave + lane < bm, "a_s LDS float past the tile");
                            if (m < M) {
                                CHECK(in && static_cast<int64_t>(off) == 4 * (kb * M + m), "a_s[%lld, %lld] address", (long long)m, (long long)kb);
                                ++sa[apw * wave + lane];
                            } else {
                                CHECK(!in, "a_s row %lld >= M read", (long long)m);
                            }
                        }
                        // per-column B scales
                        const uint64_t offb = static_cast<uint64_t>(fast_bscale_col_base(cpw, n0, N, wave, lane)) + fast_bscale_col_advance(kb, N);
                        const bool inb = access(offb, 4 * N * Kb, 4, ok);
                        CHECK(ok, "b_s offset");
                        const int64_t n = n0 + cpw * wave + lane;
                        if (lane < cpw && n < N) {
                            CHECK(inb && static_cast<int64_t>(offb) == 4 * (kb * N + n), "b_s[%lld, %lld] address", (long long)kb, (long long)n);
                            ++sbc[cpw * wave + lane];
                        } else {
                            CHECK(!inb, "b_s lane %d (column %lld) read", lane, (long long)n);
                        }
                    }
                for (int r = 0; r < arows; ++r) CHECK(sa[r] == 1, "a_s row %lld not loaded once", (long long)(m0 + r));
                for (int r = 0; r < brows; ++r) CHECK(sbc[r] == 1, "b_s column %lld not loaded once", (long long)(n0 + r));
                // 128x128 B scales: wave 0, lanes 0 and 1 (the other lanes and waves switched off)
                for (const auto& st : strides) {
                    const int64_t ext = bscale_blk_extent(N, Kb, st[0], st[1]);
                    for (int lane = 0; lane < 2; ++lane) {
                        const uint64_t off = static_cast<uint64_t>(fast_bscale_blk_base(tn, N, st[0], 0, lane)) + fast_bscale_blk_advance(kb, st[1]);
                        bool ok;
                        const bool in = access(off, 4 * ext, 4, ok);
                        CHECK(ok, "128x128 b_s offset");
                        const int64_t nb = 2 * static_cast<int64_t>(tn) + lane;
                        if (nb * kBlockK < N) {
                            CHECK(in && static_cast<int64_t>(off) == 4 * (nb * st[0] + kb * st[1]), "128x128 b_s address");
                        } else {
                            CHECK(!in, "128x128 b_s block %lld past N read", (long long)nb);
                        }
                    }
                }
            }
            // bf16 epilogue
            for (int wave = 0; wave < waves; ++wave)
                for (int p = 0; p < wr / 4; ++p)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int64_t m = fast_store_row(wr, m0, wave % wms, p, lane);
                        CHECK(m - m0 < bm, "output row outside the tile");
                        const int64_t n = fast_store_col(n0, wave / wms, lane);
                        if (m >= M) continue;
                        for (int e = 0; e < 8; ++e)
                            if (n + e < N) CHECK(++stored[m * N + n + e] == 1, "C[%lld, %lld] stored twice", (long long)m, (long long)(n + e));
                    }
        }
    for (int64_t i = 0; i < M * N; ++i) CHECK(stored[i] == 1, "C element %lld not stored", (long long)i);
    return true;
}

// Split K: slices partition the K-blocks; each slice's fp32 partial tile covers every output once.
static bool check_split(int64_t M, int64_t N, int64_t K, int bm, int wr) {
    const int wms = bm / wr, waves = 2 * wms;
    const int64_t Kb = cdiv(K, kBlockK);
    for (int64_t S = 1; S <= Kb && S <= 40; ++S) {
        int64_t next = 0;
        for (int64_t s = 0; s < S; ++s) {
            const int64_t b = split_begin(Kb, S, s), e = split_begin(Kb, S, s + 1);
            CHECK(b == next && e > b, "slice %lld of %lld: [%lld, %lld)", (long long)s, (long long)S, (long long)b, (long long)e);
            next = e;
        }
        CHECK(next == Kb, "slices end at %lld of %lld", (long long)next, (long long)Kb);
    }
    const int64_t ldp = (N + 7) / 8 * 8;
    std::vector<uint8_t> stored(static_cast<size_t>(M) * ldp, 0);
    const int mt = static_cast<int>(cdiv(M, bm)), nt = static_cast<int>(cdiv(N, kFastBN));
    for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < nt; ++tn)
            for (int wave = 0; wave < waves; ++wave)
                for (int i = 0; i < wr / 16; ++i)
                    for (int j = 0; j < 8; ++j)
                        for (int lane = 0; lane < 64; ++lane) {
                            const int64_t m = fast_partial_row(wr, static_cast<int64_t>(tm) * bm, wave % wms, i, lane);
                            const int64_t n = fast_partial_col(static_cast<int64_t>(tn) * kFastBN, wave / wms, j, lane);
                            if (m >= M || n >= N) continue;
                            CHECK(n % 4 == 0 && n + 4 <= ldp, "partial store past the padded row");
                            for (int e = 0; e < 4; ++e) CHECK(++stored[m * ldp + n + e] == 1, "partial stored twice");
                        }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) CHECK(stored[m * ldp + n] == 1, "partial (%lld, %lld) not stored", (long long)m, (long long)n);
    return true;
}

static bool check_tail_masks() {
    for (int krem = 1; krem <= kBlockK; ++krem)
        for (int lg = 0; lg < 4; ++lg)
            for (int d = 0; d < 8; ++d) {
                const uint32_t m = tail_keep_mask(krem, lg, d);
                for (int b = 0; b < 4; ++b) {
                    const bool keep = ((m >> (8 * b)) & 0xFF) == 0xFF;
                    const bool zero = ((m >> (8 * b)) & 0xFF) == 0;
                    CHECK(keep || zero, "partial byte mask");
                    CHECK(keep == (fragment_byte(lg, d) + b < krem), "krem %d lg %d d %d byte %d", krem, lg, d, b);
                }
            }
    // the fragment bytes of the four lane groups are each row byte exactly once
    std::vector<int> hit(128, 0);
    for (int lg = 0; lg < 4; ++lg)
        for (int d = 0; d < 8; ++d)
            for (int b = 0; b < 4; ++b) ++hit[fragment_byte(lg, d) + b];
    for (int i = 0; i < 128; ++i) CHECK(hit[i] == 1, "fragment byte %d", i);
    return true;
}

// ---------------------------------------------------------------------------------------------
// Thin kernel: 64 x bn tiles (bn = 32, 64, 128), 4 waves; every operand group, scale and output.
static bool check_thin(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int bn, int waves) {
    const int mt = static_cast<int>(cdiv(M, kThinBM)), nt = static_cast<int>(cdiv(N, bn));
    const int64_t Kb = cdiv(K, kBlockK);
    if (!check_tiles(mt, nt)) return false;
    const int64_t Nb = cdiv(N, kBlockK);
    const int64_t strides[2][2] = {{Kb, 1}, {1, Nb}};
    // the row groups of a tile are dealt to the waves exactly once
    {
        std::vector<int> ga(kThinBM / 8, 0), gb(bn / 8, 0);
        for (int wave = 0; wave < waves; ++wave)
            for (int p = 0; p < thin_loads(bn, waves); ++p) {
                const int gr = thin_group(bn, waves, wave, p);
                if (thin_load_is_a(bn, waves, wave, p)) {
                    CHECK(gr >= 0 && gr < kThinBM / 8, "A group %d", gr);
                    ++ga[gr];
                } else {
                    CHECK(gr >= 0 && gr < bn / 8, "B group %d", gr);
                    ++gb[gr];
                }
            }
        for (int g : ga) CHECK(g == 1, "A group dealt %d times", g);
        for (int g : gb) CHECK(g == 1, "B group dealt %d times", g);
    }
    std::vector<uint8_t> stored(static_cast<size_t>(M) * N, 0);
    for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < nt; ++tn) {
            const int64_t m0 = static_cast<int64_t>(tm) * kThinBM, n0 = static_cast<int64_t>(tn) * bn;
            const int64_t arows = M - m0 < kThinBM ? M - m0 : kThinBM;
            const int64_t brows = N - n0 < bn ? N - n0 : bn;
            for (int64_t kb = 0; kb < Kb; ++kb) {
                std::vector<uint8_t> got_a(kThinBM * 8, 0), got_b(static_cast<size_t>(bn) * 8, 0);
                for (int wave = 0; wave < waves; ++wave)
                    for (int p = 0; p < thin_loads(bn, waves); ++p) {
                        const bool is_a = thin_load_is_a(bn, waves, wave, p);
                        const int gr = thin_group(bn, waves, wave, p);
                        const int64_t rows = is_a ? arows : brows, ld = is_a ? lda : ldb;
                        const int64_t r0 = is_a ? m0 : n0, total = is_a ? M : N;
                        const int64_t range = thin_operand_range(rows, ld);
                        for (int lane = 0; lane < 64; ++lane) {
                            const uint64_t off = static_cast<uint64_t>(thin_operand_lane(gr, lane, ld)) + fast_operand_advance(kb);
                            bool ok;
                            const bool in = access(off, range, 16, ok);
                            CHECK(ok, "thin operand offset %llu (range %lld)", (unsigned long long)off, (long long)range);
                            const int r = thin_operand_row(gr, lane);
                            const int c = fast_operand_chunk(gr, lane);
                            // LDS slot: row r, position lane % 8, read by the fragments as logical
                            // chunk (lane % 8) ^ swizzle(r)
                            CHECK(thin_load_unit(bn, waves, wave, p) + lane == (is_a ? 0 : kThinBM * 8) + r * 8 + (lane & 7), "thin LDS unit");
                            CHECK(((lane & 7) ^ lds_swizzle(r)) == c, "thin LDS chunk position");
                            if (r < rows) {
                                CHECK(static_cast<int64_t>(off) == r * ld + kb * kBlockK + 16 * c, "thin operand address");
                                if (kb * kBlockK + 16 * c < K) {
                                    CHECK(in, "thin row %d chunk %d below K not read", r, c);
                                    std::vector<uint8_t>& got = is_a ? got_a : got_b;
                                    CHECK(++got[r * 8 + c] == 1, "thin row %d chunk %d loaded twice", r, c);
                                }
                            } else {
                                CHECK(!in, "thin row %d past the tile's %lld rows is read", r, (long long)rows);
                            }
                            if (in) CHECK(r0 * ld + static_cast<int64_t>(off) + 16 <= total * ld, "thin read past the operand");
                        }
                    }
                for (int r = 0; r < arows; ++r)
                    for (int c = 0; c < 8; ++c)
                        if (kb * kBlockK + 16 * c < K) CHECK(got_a[r * 8 + c] == 1, "thin A row %d chunk %d not loaded", r, c);
                for (int r = 0; r < brows; ++r)
                    for (int c = 0; c < 8; ++c)
                        if (kb * kBlockK + 16 * c < K) CHECK(got_b[r * 8 + c] == 1, "thin B row %d chunk %d not loaded", r, c);
                // A scales: wave 0, every lane (LDS float lane)
                std::vector<uint8_t> sa(kThinBM, 0), sbc(bn, 0);
                for (int lane = 0; lane < 64; ++lane) {
                    bool ok;
                    const uint64_t off = static_cast<uint64_t>(thin_ascale_base(m0, M, lane)) + fast_ascale_advance(kb, M);
                    const bool in = access(off, 4 * M * Kb, 4, ok);
                    CHECK(ok, "thin a_s offset");
                    const int64_t m = m0 + lane;
                    if (m < M) {
                        CHECK(in && static_cast<int64_t>(off) == 4 * (kb * M + m), "thin a_s[%lld, %lld] address", (long long)m, (long long)kb);
                        ++sa[lane];
                    } else {
                        CHECK(!in, "thin a_s row %lld >= M read", (long long)m);
                    }
                }
                for (int r = 0; r < arows; ++r) CHECK(sa[r] == 1, "thin a_s row %lld not loaded once", (long long)(m0 + r));
                // per-column B scales: the active lanes of the B-scale waves, each writing one LDS
                // float of the tile's bn
                for (int wave = 0; wave < waves; ++wave) {
                    if (!thin_has_bscale_load(bn, true, wave)) continue;
                    for (int lane = 0; lane < 64; ++lane) {
                        if (!((thin_bscale_lanes(bn, true) >> lane) & 1)) continue;
                        bool ok;
                        const uint64_t off = static_cast<uint64_t>(thin_bscale_col_base(bn, n0, N, wave, lane)) + fast_bscale_col_advance(kb, N);
                        const bool in = access(off, 4 * N * Kb, 4, ok);
                        CHECK(ok, "thin b_s offset");
                        const int col = thin_bscale_col(wave, lane);
                        CHECK(col < bn, "thin b_s LDS float %d outside the tile's %d", col, bn);
                        const int64_t n = n0 + col;
                        if (n < N) {
                            CHECK(in && static_cast<int64_t>(off) == 4 * (kb * N + n), "thin b_s[%lld, %lld] address", (long long)kb, (long long)n);
                            ++sbc[col];
                        } else {
                            CHECK(!in, "thin b_s column %lld >= N read", (long long)n);
                        }
                    }
                }
                for (int r = 0; r < brows; ++r) CHECK(sbc[r] == 1, "thin b_s column %lld not loaded once", (long long)(n0 + r));
                // 128x128 B scale: lane 0 of wave 3, the tile's column block
                for (const auto& st : strides) {
                    CHECK(thin_has_bscale_load(bn, false, 3) && !thin_has_bscale_load(bn, false, 2), "thin 128x128 scale wave");
                    CHECK(thin_bscale_lanes(bn, false) == 1, "thin 128x128 scale lanes");
                    bool ok;
                    const uint64_t off = static_cast<uint64_t>(thin_bscale_blk_base(n0, st[0], 0)) + fast_bscale_blk_advance(kb, st[1]);
                    const bool in = access(off, 4 * bscale_blk_extent(N, Kb, st[0], st[1]), 4, ok);
                    CHECK(ok, "thin 128x128 b_s offset");
                    const int64_t nb = n0 / kBlockK;
                    CHECK(in && static_cast<int64_t>(off) == 4 * (nb * st[0] + kb * st[1]), "thin 128x128 b_s address");
                    CHECK((n0 + brows - 1) / kBlockK == nb, "thin tile spans two column blocks");
                }
            }
            for (int wave = 0; wave < waves; ++wave)
                for (int i = 0; i < 8 / waves; ++i)
                    for (int j = 0; j < bn / 32; ++j)
                        for (int lane = 0; lane < 64; ++lane) {
                            const int64_t m = thin_store_row(m0, waves, wave % (waves / 2), i, lane);
                            const int64_t n = thin_store_col(n0, bn, wave / (waves / 2), j, lane);
                            CHECK(m - m0 < kThinBM && n - n0 < bn, "thin output outside the tile");
                            if (m >= M) continue;
                            for (int e = 0; e < 4; ++e)
                                if (n + e < N) CHECK(++stored[m * N + n + e] == 1, "thin C[%lld, %lld] stored twice", (long long)m, (long long)(n + e));
                        }
        }
    for (int64_t i = 0; i < M * N; ++i) CHECK(stored[i] == 1, "thin C element %lld not stored", (long long)i);
    return true;
}

// ---------------------------------------------------------------------------------------------
// General (float8_e4m3fnuz) kernel: 256 x 128 tiles, 8 waves of 64 x 64.
static bool check_gen(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    const int mt = static_cast<int>(cdiv(M, kGenBM)), nt = static_cast<int>(cdiv(N, kGenBN));
    const int64_t Kb = cdiv(K, kBlockK);
    if (!check_tiles(mt, nt)) return false;
    std::vector<uint8_t> stored(static_cast<size_t>(M) * N, 0);
    for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < nt; ++tn) {
            const int64_t m0 = static_cast<int64_t>(tm) * kGenBM, n0 = static_cast<int64_t>(tn) * kGenBN;
            const int64_t arows = M - m0 < kGenBM ? M - m0 : kGenBM;
            const int64_t brows = N - n0 < kGenBN ? N - n0 : kGenBN;
            for (int64_t kb = 0; kb < Kb; ++kb) {
                std::vector<uint8_t> ga(2 * 256 * 8, 0), gb(128 * 8, 0), gbd(128 * 8, 0), gbs(128, 0);  // A: once per column half (wave % 2)
                for (int wave = 0; wave < 8; ++wave)
                    for (int lane = 0; lane < 64; ++lane) {
                        bool ok;
                        // A: subtile i, two 16-byte halves
                        for (int i = 0; i < 4; ++i)
                            for (int h = 0; h < 2; ++h) {
                                const uint64_t off = static_cast<uint64_t>(gen_a_lane(wave >> 1, lane, lda)) + kb * kBlockK + 16 * h;
                                const int64_t range = gen_a_range(i, arows, lda);
                                const bool in = access(off, range, 16, ok);
                                CHECK(ok, "gen A offset");
                                const int r = gen_a_row(wave >> 1, i, lane);
                                const int c = 2 * (lane >> 4) + h;
                                if (r < arows) {
                                    CHECK(static_cast<int64_t>(off) == (r - gen_a_first_row(i)) * lda + kb * kBlockK + 16 * c, "gen A address");
                                    if (kb * kBlockK + 16 * c < K) {
                                        CHECK(in, "gen A row %d not read", r);
                                        CHECK(++ga[(wave & 1) * 2048 + r * 8 + c] == 1, "gen A chunk twice");
                                    }
                                } else {
                                    CHECK(!in, "gen A row %d past the tile read", r);
                                }
                                if (in) CHECK((m0 + gen_a_first_row(i)) * lda + static_cast<int64_t>(off) + 16 <= M * lda, "gen A past the operand");
                            }
                        // A scales
                        for (int i = 0; i < 4; ++i) {
                            const uint64_t off = static_cast<uint64_t>(gen_ascale_base(m0, wave >> 1, i, lane, M)) + 4 * kb * M;
                            const bool in = access(off, 4 * M * Kb, 4, ok);
                            CHECK(ok, "gen a_s offset");
                            const int64_t m = m0 + gen_a_row(wave >> 1, i, lane);
                            CHECK(in == (m < M), "gen a_s row %lld", (long long)m);
                            if (in) CHECK(static_cast<int64_t>(off) == 4 * (kb * M + m), "gen a_s address");
                        }
                        // per-column B scales: one per thread of the first 128, staged in LDS
                        {
                            const int tid = 64 * wave + lane;
                            const uint64_t off = static_cast<uint64_t>(gen_bscale_tile_base(n0, N, tid)) + 4 * kb * N;
                            const bool in = access(off, 4 * N * Kb, 4, ok);
                            CHECK(ok, "gen b_s offset");
                            const int64_t n = n0 + tid;
                            if (tid < kGenBN && n < N) {
                                CHECK(in && static_cast<int64_t>(off) == 4 * (kb * N + n), "gen b_s[%lld, %lld] address", (long long)kb, (long long)n);
                                ++gbs[tid];
                            } else {
                                CHECK(!in, "gen b_s thread %d (column %lld) read", tid, (long long)n);
                            }
                        }
                        // B through registers (partial K-block) and straight into LDS
                        const int tid = 64 * wave + lane;
                        for (int p = 0; p < 2; ++p) {
                            const uint64_t off = static_cast<uint64_t>(gen_b_lane(tid, ldb)) + kb * kBlockK;
                            const bool in = access(off, gen_b_range(p, brows, ldb), 16, ok);
                            CHECK(ok, "gen B offset");
                            const int r = gen_b_row(tid, p);
                            if (r < brows) {
                                if (kb * kBlockK + 16 * (tid & 7) < K) CHECK(in && ++gb[r * 8 + (tid & 7)] == 1, "gen B row %d", r);
                            } else {
                                CHECK(!in, "gen B row %d past the tile read", r);
                            }
                        }
                        for (int q = 0; q < 2; ++q) {
                            const uint64_t off = static_cast<uint64_t>(gen_bdma_lane(wave, lane, ldb)) + kb * kBlockK;
                            const bool in = access(off, gen_bdma_range(q, brows, ldb), 16, ok);
                            CHECK(ok, "gen B DMA offset");
                            const int r = gen_bdma_row(wave, q, lane);
                            const int c = (lane & 7) ^ (lane >> 3);
                            CHECK(c == ((lane & 7) ^ (r & 7)), "gen B LDS chunk position");
                            if (r < brows) {
                                // the direct load serves full K-blocks only
                                if ((kb + 1) * kBlockK <= K) CHECK(in && ++gbd[r * 8 + c] == 1, "gen B DMA row %d", r);
                            } else {
                                CHECK(!in, "gen B DMA row %d past the tile read", r);
                            }
                        }
                    }
                for (int r = 0; r < arows; ++r)
                    for (int c = 0; c < 8; ++c)
                        if (kb * kBlockK + 16 * c < K) CHECK(ga[r * 8 + c] == 1 && ga[2048 + r * 8 + c] == 1, "gen A row %d chunk %d", r, c);
                for (int r = 0; r < brows; ++r) {
                    for (int c = 0; c < 8; ++c) {
                        if (kb * kBlockK + 16 * c < K) CHECK(gb[r * 8 + c] == 1, "gen B row %d chunk %d", r, c);
                        if ((kb + 1) * kBlockK <= K) CHECK(gbd[r * 8 + c] == 1, "gen B DMA row %d chunk %d", r, c);
                    }
                    CHECK(gbs[r] == 1, "gen b_s column %lld not loaded once", (long long)(n0 + r));
                }
            }
            for (int wave = 0; wave < 8; ++wave)
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j)
                        for (int lane = 0; lane < 64; ++lane) {
                            const int64_t m = m0 + gen_a_row(wave >> 1, i, lane);
                            const int64_t n = gen_col(n0, wave & 1, j, lane);
                            if (m >= M) continue;
                            for (int e = 0; e < 4; ++e)
                                if (n + e < N) CHECK(++stored[m * N + n + e] == 1, "gen C stored twice");
                        }
        }
    for (int64_t i = 0; i < M * N; ++i) CHECK(stored[i] == 1, "gen C element %lld not stored", (long long)i);
    return true;
}

// ---------------------------------------------------------------------------------------------
// quantize_lhs scale stores (units of 64 rows of one K-block, 16 teams x 4 rows per unit).
static bool check_lhs_scales(int64_t M, int64_t K) {
    const int64_t Kb = cdiv(K, kBlockK);
    const int rows_per_team = 4;
    const int64_t units = cdiv(M, 16 * rows_per_team) * Kb;
    std::vector<uint8_t> w(static_cast<size_t>(M) * Kb, 0);
    for (int64_t u = 0; u < units; ++u) {
        int64_t rb, kb;
        lhs_unit(u, Kb, rb, kb);
        CHECK(kb >= 0 && kb < Kb, "unit K-block");
        for (int team = 0; team < 16; ++team)
            for (int r = 0; r < rows_per_team; ++r) {
                const int64_t m = lhs_row(rb, rows_per_team, r, team);
                if (!row_stored(m, M)) continue;  // the kernel's store predicate
                const int64_t idx = colmajor_index(kb, M, m);
                CHECK(m < M && idx >= 0 && idx < M * Kb, "a_s store of row %lld (index %lld)", (long long)m, (long long)idx);
                CHECK(++w[idx] == 1, "a_s[%lld] stored twice", (long long)idx);
            }
    }
    for (int64_t i = 0; i < M * Kb; ++i) CHECK(w[i] == 1, "a_s[%lld] not stored", (long long)i);
    return true;
}

// ---------------------------------------------------------------------------------------------
// The thin kernel's LDS pipeline, simulated wave by wave for every depth it instantiates and every
// K-block count up to 40 (with and without a partial last block, which runs as a step of its own),
// with L loads per wave per block (the kernel's 3..7 operand and scale loads). The iterations
// mirror the kernel's three loops: blocks_per_step blocks while that many full blocks remain, then
// single full blocks, then the partial one. Loads complete in issue order (what vmcnt counts); the
// wait of an iteration lets at most thin_wait_later * L of them stay outstanding. Checked: the
// blocks an iteration multiplies have all landed; a block is issued into a stage only when that
// stage's previous block was multiplied before the iteration's barrier; the vmcnt immediate fits
// its 6 bits; every block is issued once and multiplied once, in order.
static bool check_thin_pipeline() {
    for (int stages : {2, 3, 4, 6, 8, 12})
        for (int L = 3; L <= 8; ++L) {
            const int nb = thin_blocks_per_step(stages), ahead = thin_ahead(stages);
            CHECK(nb >= 1 && ahead >= nb && L * (ahead - 1) <= 63, "stages %d: nb %d ahead %d", stages, nb, ahead);
            for (int Kb = 1; Kb <= 40; ++Kb)
                for (int partial = 0; partial < 2; ++partial) {
                    const int Kb_full = partial ? Kb - 1 : Kb;
                    std::vector<int> owner(stages, -1);      // block resident in each stage
                    std::vector<int> done_mult(Kb, 0), issued(Kb, 0);
                    std::vector<int> fifo;                   // outstanding loads (block of each), oldest first
                    std::vector<int> landed(Kb, 0);          // loads of the block completed
                    std::vector<int> freed_at_barrier;       // blocks multiplied since the last barrier
                    auto issue = [&](int b) -> bool {
                        const int st = thin_stage_of(stages, b);
                        CHECK(st >= 0 && st < stages, "stage of block %d", b);
                        CHECK(owner[st] == -1 || done_mult[owner[st]] == 2,
                              "stages %d Kb %d: block %d issued into stage %d, still holding block %d", stages, Kb, b, st, owner[st]);
                        CHECK(!issued[b], "block %d issued twice", b);
                        owner[st] = b;
                        issued[b] = 1;
                        for (int l = 0; l < L; ++l) fifo.push_back(b);
                        return true;
                    };
                    for (int b = 0; b < ahead; ++b)
                        if (b < Kb && !issue(b)) return false;
                    int next = 0;  // next block to multiply
                    auto step = [&](int kb, int n) -> bool {
                        const int later = thin_wait_later(stages, kb, n, Kb);
                        const int allowed = later > 0 ? later * L : 0;
                        CHECK(allowed <= 63, "vmcnt %d", allowed);
                        while (static_cast<int>(fifo.size()) > allowed) {
                            const int b = fifo.front();
                            fifo.erase(fifo.begin());
                            int left = 0;
                            for (int x : fifo) left += x == b;
                            if (left == 0) landed[b] = 1;
                        }
                        // barrier: blocks multiplied before it no longer hold their stages
                        for (int b : freed_at_barrier) done_mult[b] = 2;
                        freed_at_barrier.clear();
                        for (int q = 0; q < n; ++q)
                            if (kb + ahead + q < Kb && !issue(kb + ahead + q)) return false;
                        for (int q = 0; q < n; ++q) {
                            const int b = kb + q;
                            CHECK(b == next, "block %d multiplied out of order (expected %d)", b, next);
                            CHECK(issued[b] && landed[b], "stages %d Kb %d L %d: block %d multiplied before its loads landed",
                                  stages, Kb, L, b);
                            CHECK(owner[thin_stage_of(stages, b)] == b, "block %d not in its stage", b);
                            done_mult[b] = 1;
                            freed_at_barrier.push_back(b);
                            ++next;
                        }
                        return true;
                    };
                    int kb = 0;
                    for (; kb + nb <= Kb_full; kb += nb)
                        if (!step(kb, nb)) return false;
                    for (; kb < Kb_full; ++kb)
                        if (!step(kb, 1)) return false;
                    if (Kb_full < Kb && !step(Kb - 1, 1)) return false;
                    CHECK(next == Kb, "stages %d Kb %d: %d of %d blocks multiplied", stages, Kb, next, Kb);
                    CHECK(fifo.empty(), "loads left in flight at the end");
                }
        }
    return true;
}

// ---------------------------------------------------------------------------------------------
// quantize_lhs in row strips (K % 16 == 0), every pieces-per-thread count the library launches:
// each input piece of 8 columns is read once and lands in the LDS slot of its (row, K-block) group,
// a group's 16 pieces sit in one aligned 16-lane row of a wave, each 16-byte output piece is written
// once from the LDS bytes its two input pieces encoded, each scale once from its group's LDS slot,
// and no row >= M and no column >= K is read or written.
static bool check_lhs_strips(int64_t M, int64_t K) {
    if (K % 16 != 0) return true;  // such shapes run the tile kernel
    const int64_t Kb = cdiv(K, kBlockK);
    for (int nl : {1, 2, 4, 8, 16}) {
        const StripShape sh = strip_shape(M, Kb, nl);
        CHECK(sh.g >= 1 && sh.g <= 32 && sh.rows >= 1, "strip shape nl=%d: rows %d g %d", nl, sh.rows, sh.g);
        CHECK(sh.rows * 16 * sh.g <= kStripThreads * nl && sh.loads <= nl, "strip of nl=%d overflows", nl);
        CHECK(sh.chunks * sh.g >= Kb && (sh.chunks - 1) * sh.g < Kb, "strip chunks nl=%d", nl);
        std::vector<uint8_t> rd(static_cast<size_t>(M) * (K / 8), 0), wr(static_cast<size_t>(M) * (K / 16), 0);
        std::vector<uint8_t> sc(static_cast<size_t>(M) * Kb, 0);
        for (int64_t u = 0; u < sh.units; ++u) {
            int64_t strip, chunk;
            strip_unit(u, sh.chunks, strip, chunk);
            const int64_t m0 = strip * sh.rows, kb0 = chunk * sh.g, c0 = kb0 * kBlockK;
            CHECK(kb0 < Kb && m0 < M, "strip unit %lld outside the tensor", (long long)u);
            for (int t = 0; t < kStripThreads; ++t) {
                for (int j = 0; j < nl; ++j) {
                    const int p = t + kStripThreads * j;
                    int64_t m, c;
                    if (!strip_piece(p, sh, m0, c0, M, K, m, c)) continue;
                    CHECK(m >= 0 && m < M && c >= 0 && c + 8 <= K && c % 8 == 0, "strip read row %lld col %lld", (long long)m, (long long)c);
                    CHECK(++rd[static_cast<size_t>(m * (K / 8) + c / 8)] == 1, "strip piece read twice");
                    // the group of 16 aligned lanes: one row, one K-block, lane t % 16 at piece t % 16
                    CHECK(c / kBlockK == kb0 + (p % (16 * sh.g)) / 16 && (c % kBlockK) / 8 == (t & 15) &&
                              m == m0 + (p >> 4) / sh.g,
                          "strip group of lane %d", t);
                    CHECK(p < kStripThreads * nl && (p >> 4) < kStripThreads * nl / 16, "strip LDS slot");
                }
                for (int i = 0; i < (nl + 1) / 2; ++i) {
                    const int q = t + kStripThreads * i;
                    int64_t m, c;
                    if (!strip_out_piece(q, sh, m0, c0, M, K, m, c)) continue;
                    CHECK(m >= 0 && m < M && c >= 0 && c + 16 <= K && c % 16 == 0, "strip store row %lld col %lld", (long long)m, (long long)c);
                    CHECK(++wr[static_cast<size_t>(m * (K / 16) + c / 16)] == 1, "strip piece stored twice");
                    CHECK(16 * (q + 1) <= 8 * kStripThreads * nl, "strip LDS read past the codes");
                    // LDS bytes 16 q .. 16 q + 15 hold the codes of input pieces 2 q and 2 q + 1
                    int64_t ma, ca, mb, cb;
                    const bool ia = strip_piece(2 * q, sh, m0, c0, M, K, ma, ca);
                    const bool ib = strip_piece(2 * q + 1, sh, m0, c0, M, K, mb, cb);
                    CHECK(ia && ib && ma == m && mb == m && ca == c && cb == c + 8, "strip store of piece %d", q);
                }
            }
            for (int i = 0; i < sh.rows * sh.g; ++i) {
                int64_t kb, m;
                if (!strip_scale(i, sh, m0, kb0, M, Kb, kb, m)) continue;
                const int64_t idx = colmajor_index(kb, M, m);
                CHECK(m < M && kb < Kb && idx >= 0 && idx < M * Kb, "strip a_s store of row %lld (index %lld)", (long long)m, (long long)idx);
                CHECK(++sc[static_cast<size_t>(idx)] == 1, "strip a_s[%lld] stored twice", (long long)idx);
                CHECK((i % sh.rows) * sh.g + i / sh.rows == (m - m0) * sh.g + (kb - kb0), "strip scale slot");
            }
        }
        for (size_t i = 0; i < rd.size(); ++i) CHECK(rd[i] == 1, "strip piece %zu not read (nl=%d)", i, nl);
        for (size_t i = 0; i < wr.size(); ++i) CHECK(wr[i] == 1, "strip piece %zu not stored (nl=%d)", i, nl);
        for (size_t i = 0; i < sc.size(); ++i) CHECK(sc[i] == 1, "strip a_s[%zu] not stored (nl=%d)", i, nl);
    }
    return true;
}

int main(int argc, char** argv) {
    if (!check_tail_masks()) return 1;
    if (!check_thin_pipeline()) return 1;
    for (int a = 1; a + 2 < argc; a += 3) {
        const int64_t M = std::atoll(argv[a]), N = std::atoll(argv[a + 1]), K = std::atoll(argv[a + 2]);
        const int64_t ld = (K + 15) / 16 * 16;  // the GEMMs' 16-byte row rule
        bool ok = true;
        for (const auto& t : {std::pair<int, int>{kFastBM, 64}, {kFastBMSmall, 64}, {kFastBMSmall, 32}})
            ok = ok && check_fast(M, N, K, ld, ld, t.first, t.second) &&
                 check_fast(M, N, K, ld + 16, ld + 48, t.first, t.second) && check_split(M, N, K, t.first, t.second);
        for (int bn : {32, 64, 128})
            for (int waves : {4, 8}) {
                if (waves == 8 && bn < 64) continue;  // 8-wave tiles are 64 or 128 columns wide
                ok = ok && check_thin(M, N, K, ld, ld, bn, waves) && check_thin(M, N, K, ld + 16, ld + 48, bn, waves);
            }
        ok = ok && check_gen(M, N, K, ld, ld) && check_lhs_scales(M, K) && check_lhs_strips(M, K);
        std::printf("%s M=%lld N=%lld K=%lld\n", ok ? "ok" : "FAILED", (long long)M, (long long)N, (long long)K);
        if (!ok) return 1;
    }
    return g_fail;
}
