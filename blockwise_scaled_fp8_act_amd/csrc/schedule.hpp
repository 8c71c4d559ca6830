// GEMM schedule: which kernel and tiles a problem takes, whether K is split, and the thin kernel's
// pipeline depth. Plain C++ (no HIP): the library calls it on the host before every GEMM launch,
// and tests/schedule_check.cpp compiles the same header with the host compiler to check the rules
// shape by shape.
//
// The rules, from measurements on MI355X (256 CUs; settled clock):
//   * 256 x 256 tiles (8 waves of 64 x 128, two per SIMD) run the K-loop fastest and are kept
//     whenever they give every CU a tile; a problem with at most half as many 256-row tiles as CUs,
//     or with M <= 128 (a 256-row tile would be at least half empty), takes 128 x 256 tiles (8
//     waves of 32 x 128; twice the tiles);
//   * when the 128-row tiles would fill at most half the CUs, the problem takes the thin kernel's
//     64-row tiles, the widest (128, 64 or 32 columns) that still occupy three quarters of the CUs,
//     in 8 waves of 16-row blocks when the grid is at most one workgroup per CU: the loop is
//     latency-bound, so a wider tile's extra work per barrier and a second wave per SIMD beat more
//     workgroups (settled clock: 256 x 4096 x 4096 13.9 us in 64 x 64 tiles of 8 waves against
//     17.0 in twice as many 64 x 32; 192 rows 13.8 in 192 such tiles against 16.9 in 384 of 64 x 32;
//     160 x 4096 x 8192 24.0 against 28.1; 384 rows 19.1 in 192 tiles of 64 x 128 against 19.5 in
//     384 of 64 x 64; 768 rows 26.9 in 64 x 128 tiles (4 waves) against 29.7; M = 128, where 64 x 64
//     tiles would leave half the CUs idle: 11.7 in 64 x 32 against 13.6; 1024 x 4096 x 4096: 27.3
//     us in 64 x 128 thin tiles, 32.9 in 128 x 256 tiles; 1536 rows: 38.0 against 33.3);
//   * only when those are fewer than half the CUs and K is longer than 64 blocks does K get split
//     instead (at 64 x 1024 x 8192 the thin kernel's 32 workgroups still beat 64 slices, 27
//     against 32 us): S workgroups per 128- or 256-row tile, whose fp32 partial tiles (written,
//     then read by the sum) and second launch pay off when the tiles leave most CUs idle; the
//     slices always fit in one round;
//   * the thin kernel runs the deepest pipeline (12, 8, 6, 4, 3 or 2 LDS stages) whose LDS still
//     lets every workgroup of the grid be resident at once; from four stages on it multiplies two
//     K-blocks per barrier, from twelve four. Its loop is latency-bound (one or two 4-wave
//     workgroups per CU: at 128 x 4096 x 4096 it takes as long with its operand loads pointed at
//     an empty buffer), so blocks in flight and work per barrier matter more than extra workgroups
//     per CU (128 x 4096 x 4096, 256 workgroups, settled clock: 15.8 us with three stages, 15.9
//     with four, 12.4 with eight, 11.7 with twelve; 64 x 1024 x 8192: 21.1 with eight, 19.3 with
//     twelve). The deepest pipeline that fits a workgroup's LDS (thin_max_stages) bounds what a
//     forced schedule may ask for.
#pragma once

#include <stdint.h>

#include <initializer_list>

#include "geometry.hpp"

namespace bsfp8 {

// Schedule of a GEMM: the tile height bm -- 256 or 128 rows (the fast kernel) or 64 (the thin
// kernel, whose tiles are bn = 32, 64 or 128 columns wide; bn is 0 for the fast kernel's 256) --
// and the K split of a fast-kernel GEMM whose output tiles cannot fill the chip: S workgroups per
// tile each multiply a range of K-blocks into an fp32 partial tile (rows of ldp floats, ldp = N
// rounded up to 8), and a second kernel sums the S partials into C. S == 1: no split. bytes: the
// fp32 workspace it needs.
struct SplitPlan {
    int S;
    int64_t ldp;
    int64_t bytes;
    int bm;
    int bn;
    int stages = 0;  // the thin kernel's LDS stages; 0: sched::thin_stages at launch
    int waves = 0;   // the thin kernel's waves per workgroup (4 or 8); 0: sched::thin_waves at launch
};

namespace sched {

constexpr int64_t kLdsPerCu = 160 * 1024;  // LDS bytes of a gfx950 compute unit

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// quantize_lhs in row strips: 16-byte input pieces per thread (1, 2, 4, 8 or 16; the strip height
// follows) for an M x (128 Kb) activation. A workgroup of 16 pieces per thread holds 66 KB of LDS
// (two per CU), one of 8 or fewer at most four per CU (32 waves of 8-wave workgroups). The rules,
// from a sweep on MI355X:
//   * when some strip size gives every CU at least two workgroups and still lets the whole grid be
//     resident at once, the largest such size (4096 x 4096: 8 pieces, 9.8 us, against 11.0 us with
//     4 and 10.8 us in tiles; 8192 x 4096: 16 pieces, 18.7 us, against 19.4 with 4);
//   * when every size needs more rounds of workgroups than one, 4 pieces: small workgroups that
//     come and go keep the HBM busier than big ones that wait for whole strips (16384 x 4096:
//     35.0 us, against 36.2 with 16 and 39.7 in tiles; 32768 x 4096: 66.5 against 69.9);
//   * when even one piece per thread leaves CUs with fewer than two workgroups, one piece (the
//     most workgroups; these shapes take a few microseconds whatever the choice).
inline int strip_resident(int nl) {
    // LDS of the strip kernel: 8 code bytes per piece, one fp32 scale per 16 pieces
    const int64_t lds = static_cast<int64_t>(geom::kStripThreads) * nl * 8 + geom::kStripThreads * nl / 16 * 4;
    const int64_t by_lds = kLdsPerCu / lds;
    return static_cast<int>(by_lds < 4 ? by_lds : 4);
}
inline int lhs_strip_loads(int64_t M, int64_t Kb, int cus) {
    for (const int nl : {16, 8, 4, 2, 1}) {
        const int64_t u = geom::strip_shape(M, Kb, nl).units;
        if (u >= 2 * static_cast<int64_t>(cus) && u <= static_cast<int64_t>(strip_resident(nl)) * cus) return nl;
    }
    return geom::strip_shape(M, Kb, 1).units < 2 * static_cast<int64_t>(cus) ? 1 : 4;
}

// The fast kernel's tile height for M x N.
inline int fast_bm(int64_t M, int64_t N, int cus) {
    const int64_t tiles256 = cdiv(M, geom::kFastBM) * cdiv(N, geom::kFastBN);
    return (M <= geom::kFastBMSmall || 2 * tiles256 <= cus) ? geom::kFastBMSmall : geom::kFastBM;
}

// The thin kernel's tile width for M x N.
inline int thin_bn(int64_t M, int64_t N, int cus) {
    for (const int bn : {128, 64})
        if (4 * cdiv(M, geom::kThinBM) * cdiv(N, bn) >= 3 * static_cast<int64_t>(cus)) return bn;
    return 32;
}

// The automatic K split of the fast kernel's tiles of height plan.bm.
inline void fast_split(SplitPlan& plan, int64_t M, int64_t N, int64_t K, int cus, int64_t max_bytes) {
    const int64_t tiles = cdiv(M, plan.bm) * cdiv(N, geom::kFastBN);
    const int64_t Kb = cdiv(K, geom::kBlockK);
    if (M > 512 || 4 * tiles > cus) return;
    int64_t S = cus / tiles;  // one round of workgroups
    if (M <= 64) {
        if (S > Kb) S = Kb;
    } else {
        if (Kb <= 10) return;  // short K: the slice overhead outweighs the idle CUs
        if (S > Kb / 2) S = Kb / 2;
        if (S > (M <= 256 ? 12 : 4)) S = M <= 256 ? 12 : 4;
    }
    const int64_t ldp = (N + 7) / 8 * 8;
    const int64_t slice_bytes = M * ldp * 4;
    if (S * slice_bytes > max_bytes) S = max_bytes / slice_bytes;
    if (S > 65535) S = 65535;
    if (S < 2) return;
    plan.S = static_cast<int>(S);
    plan.ldp = ldp;
    plan.bytes = S * slice_bytes;
}

// LDS stages of the thin kernel for a grid of wgs workgroups of tile width bn: the deepest of 4, 3
// and 2 that keeps the whole grid resident (2 when none does).
// The deepest instantiated pipeline (2, 3, 4, 6, 8 or 12 stages) whose LDS fits one workgroup.
inline int thin_max_stages(int bn, bool per_col) {
    const int64_t stage_bytes = 16 * static_cast<int64_t>(geom::thin_stage_units(bn, per_col));
    for (const int st : {12, 8, 6, 4, 3})
        if (st * stage_bytes <= kLdsPerCu) return st;
    return 2;
}

// The thin kernel's waves per workgroup: 8 (16-row waves, two per SIMD) for 64- and 128-column
// tiles when the grid is at most one workgroup per CU, else 4 (768 x 4096 x 4096, 384 workgroups of
// 64 x 128: 29.7 us in 8 waves, 26.8 in 4).
inline int thin_waves(int bn, int64_t wgs, int cus) { return bn >= 64 && wgs <= static_cast<int64_t>(cus) ? 8 : 4; }

inline int thin_stages(int bn, bool per_col, int64_t wgs, int cus) {
    const int64_t stage_bytes = 16 * static_cast<int64_t>(geom::thin_stage_units(bn, per_col));
    for (const int st : {12, 8, 6, 4, 3})
        if (wgs <= static_cast<int64_t>(cus) * (kLdsPerCu / (st * stage_bytes))) return st;
    return 2;
}

}  // namespace sched

// The automatic schedule. fnuz (the general kernel): one 256 x 128 tile per workgroup, never split.
inline SplitPlan gemm_split_plan(int64_t M, int64_t N, int64_t K, bool fnuz, int cus, int64_t max_bytes) {
    SplitPlan plan{1, 0, 0, geom::kFastBM, 0};
    if (fnuz || M <= 0 || N <= 0 || K <= 0) return plan;
    plan.bm = sched::fast_bm(M, N, cus);
    if (2 * sched::cdiv(M, geom::kFastBMSmall) * sched::cdiv(N, geom::kFastBN) <= cus) {
        const int bn = sched::thin_bn(M, N, cus);
        const int64_t wgs = sched::cdiv(M, geom::kThinBM) * sched::cdiv(N, bn);
        if (2 * wgs >= cus || sched::cdiv(K, geom::kBlockK) <= 64) {
            plan.bm = geom::kThinBM;
            plan.bn = bn;
            return plan;
        }
    }
    sched::fast_split(plan, M, N, K, cus, max_bytes);
    return plan;
}

// A schedule chosen by the caller, so tests and sweeps can run any schedule on any shape: bm 64 --
// the thin kernel with tile width bn (32, 64 or 128; other values: automatic), never split; bm 256
// or 128 -- the fast kernel with that tile height and its automatic split; bm 0 -- automatic (its
// thin width may be set by bn). S > 0 sets the slice count (clamped to the K-block count and to
// max_bytes of workspace; below two: no split); a split runs on the fast kernel.
inline SplitPlan gemm_split_plan_forced(int64_t M, int64_t N, int64_t K, bool fnuz, int cus, int S, int bm, int bn,
                                        int64_t max_bytes) {
    SplitPlan plan = gemm_split_plan(M, N, K, fnuz, cus, max_bytes);
    if (fnuz || M <= 0 || N <= 0 || K <= 0) return plan;
    const bool bn_ok = bn == 32 || bn == 64 || bn == 128;
    if (bm == geom::kThinBM) return SplitPlan{1, 0, 0, geom::kThinBM, bn_ok ? bn : sched::thin_bn(M, N, cus)};
    const bool fast_forced = bm == geom::kFastBM || bm == geom::kFastBMSmall;
    if (fast_forced || (S >= 2 && plan.bm == geom::kThinBM)) {
        plan = SplitPlan{1, 0, 0, fast_forced ? bm : sched::fast_bm(M, N, cus), 0};
        sched::fast_split(plan, M, N, K, cus, max_bytes);
    } else if (plan.bm == geom::kThinBM && bn_ok) {
        plan.bn = bn;
    }
    if (S <= 0 || plan.bm == geom::kThinBM) return plan;
    plan.S = 1;
    plan.ldp = 0;
    plan.bytes = 0;
    const int64_t Kb = sched::cdiv(K, geom::kBlockK);
    const int64_t ldp = (N + 7) / 8 * 8;
    const int64_t slice_bytes = M * ldp * 4;
    int64_t s = S > Kb ? Kb : S;
    if (s * slice_bytes > max_bytes) s = max_bytes / slice_bytes;
    if (s > 65535) s = 65535;
    if (s < 2) return plan;
    plan.S = static_cast<int>(s);
    plan.ldp = ldp;
    plan.bytes = s * slice_bytes;
    return plan;
}

// Column split of a GEMM whose 256 x 256 tiles end in a partial round (4096 x 5120 x 5120: 320 tiles,
// a second round of 64 on a quarter of the CUs): the first n1 columns (whole tile columns whose
// tiles fill whole rounds) run as one GEMM; the last N - n1, whose tiles would fill at most a
// quarter of the CUs, run as a second with K split in at least 4 so its slices fill the chip
// (`tail`). A tile of a sparse last round runs faster than one of a full round (less contention, a
// higher clock), which the split gives back: measured at the settled clock, 4096 x 5120 x 5120
// 125 -> 118 us and 4096 x 5120 x 4096 103 -> 100 us with 4 slices, but 8192 x 5120 x 5120 (a
// tail of 128 tiles in 2 slices) 195 -> 207 us, hence the quarter. Only where the B scales are
// 128 x 128 blocks (an offset of n1 / 128 blocks addresses the tail's) and the automatic plan is
// unsplit 256-row tiles. n1 == 0: no column split.
struct ColumnSplit {
    int64_t n1;
    SplitPlan tail;
};
inline ColumnSplit gemm_column_split(int64_t M, int64_t N, int64_t K, int cus, int64_t max_bytes) {
    const ColumnSplit none{0, SplitPlan{1, 0, 0, geom::kFastBM, 0}};
    const SplitPlan plan = gemm_split_plan(M, N, K, false, cus, max_bytes);
    if (plan.bm != geom::kFastBM || plan.S != 1) return none;
    const int64_t mt = sched::cdiv(M, geom::kFastBM), nt = sched::cdiv(N, geom::kFastBN);
    const int64_t tiles = mt * nt;
    if (tiles <= cus || tiles % cus == 0) return none;
    int64_t nt1 = nt - 1;
    while (nt1 >= 1 && (mt * nt1) % cus != 0) --nt1;
    if (nt1 < 1) return none;
    const int64_t tail_tiles = mt * (nt - nt1);
    if (4 * tail_tiles > cus) return none;
    const int64_t n1 = nt1 * geom::kFastBN;
    const int S = static_cast<int>(cus / tail_tiles);
    const SplitPlan tail = gemm_split_plan_forced(M, N - n1, K, false, cus, S, geom::kFastBM, 0, max_bytes);
    if (tail.S < 4 || tail.bm != geom::kFastBM) return none;
    // Worth it only when the K-blocks the split takes off the tail's critical path (~1.9 us each
    // for a 256 x 256 tile at the settled clock) outweigh the partial tiles' traffic (S fp32 slices
    // written and read, bf16 C written; ~5 TB/s).
    const double saved_us = static_cast<double>(sched::cdiv(K, geom::kBlockK)) * (tail.S - 1) / tail.S * 1.9;
    const double sum_us = static_cast<double>(M) * static_cast<double>(N - n1) * (8.0 * tail.S + 2.0) / 5e6;
    if (saved_us < sum_us) return none;
    return ColumnSplit{n1, tail};
}

}  // namespace bsfp8
