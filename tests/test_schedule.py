"""CPU check of the GEMM schedule rules (csrc/schedule.hpp, compiled with the host compiler): which
kernel and tiles each shape takes, when K is split, and the thin kernel's pipeline depth -- for the
workloads, the ROCm page's GEMM table shapes, the rule boundaries and the forced schedules the
tests and sweeps use. 256 compute units (MI355X) unless stated."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_act_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "schedule_check.cpp")
CUS = 256
MAXB = 256 << 20  # the library's workspace bound for a split


@pytest.fixture(scope="module")
def sched(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, SRC, "-o", exe], check=True)

    def ask(queries):
        r = subprocess.run([exe], input="\n".join(queries) + "\n", capture_output=True, text=True, check=True)
        return [tuple(int(v) for v in ln.split()) for ln in r.stdout.strip().split("\n")]
    return ask


def _plans(sched, shapes, fnuz=0, cus=CUS):
    return sched([f"plan {M} {N} {K} {fnuz} {cus} {MAXB}" for (M, N, K) in shapes])


# (M, N, K) -> (S, bm, bn): bm 256 / 128 the fast kernel, 64 the thin kernel (tile width bn)
EXPECTED = {
    (4096, 4096, 4096): (1, 256, 0),     # the bench step: one 256 x 256 tile per CU
    (8192, 4096, 4096): (1, 256, 0),     # training-step forward / dgrad: two rounds
    (4096, 4096, 8192): (1, 256, 0),     # weight gradient over 8192 tokens
    (16384, 5120, 5120): (1, 256, 0),    # outlier workload
    (4096, 5120, 5120): (1, 256, 0),     # 320 tiles: more than the CUs
    (2048, 4096, 4096): (1, 128, 0),     # 128 tiles of 256 rows -> 256 of 128 rows
    (1536, 4096, 4096): (1, 128, 0),     # 192 tiles of 128 rows: more than half the CUs
    (2048, 8192, 4096): (1, 256, 0),
    (1024, 4096, 4096): (1, 64, 128),    # 128 tiles of 128 rows, half the CUs: thin, 512 of 64 x 128
    (512, 4096, 4096): (1, 64, 128),     # 64 x 128: 256 tiles, one per CU
    (256, 4096, 4096): (1, 64, 64),      # 64 x 128 would leave CUs idle: 64 x 64, 256 tiles
    (384, 4096, 4096): (1, 64, 128),     # 192 tiles of 64 x 128: three quarters of the CUs
    (192, 4096, 4096): (1, 64, 64),      # 192 tiles of 64 x 64
    (160, 4096, 8192): (1, 64, 64),
    (128, 4096, 4096): (1, 64, 32),      # no width gives two per CU: the narrowest
    (130, 5120, 1280): (1, 64, 64),      # tail-masking workload: 240 tiles of 64 x 64
    (2, 512, 128): (1, 64, 32),          # smallest workload
    (64, 1024, 8192): (1, 64, 32),       # 32 thin tiles, K = 64 blocks: still thin
    (64, 1024, 8320): (64, 128, 0),      # K = 65 blocks: split, 4 tiles x 64 slices = one round
    (300, 520, 704): (1, 64, 32),
}


def test_automatic_schedule(sched):
    shapes = list(EXPECTED)
    got = _plans(sched, shapes)
    for sh, g in zip(shapes, got):
        assert g[:3] == EXPECTED[sh], (sh, g)


def test_split_workspace_is_slices_of_padded_rows(sched):
    (S, bm, bn, nbytes), = _plans(sched, [(64, 1000, 16384)])
    assert bm == 128 and bn == 0 and S == 64
    assert nbytes == S * 64 * 1000 * 4  # rows padded to 8 floats: 1000 already is
    (S2, _, _, nbytes2), = _plans(sched, [(50, 1001, 16384)])
    assert nbytes2 == S2 * 50 * 1008 * 4


def test_fnuz_and_empty_problems_never_split(sched):
    for g in _plans(sched, [(128, 4096, 4096), (2, 512, 128)], fnuz=1) + _plans(sched, [(0, 5, 5), (5, 0, 5), (5, 5, 0)]):
        assert g[:3] == (1, 256, 0)


def test_thin_kernel_boundary(sched):
    """The thin kernel exactly when the 128-row tiles would fill at most half the CUs (N = 4096:
    16 column tiles, so at most cus / 32 row tiles), here and on a chip with 128 CUs."""
    for cus in (256, 128):
        last = cus // 32 * 128  # the most rows whose 128-row tiles fill at most half the CUs
        below, at = _plans(sched, [(last, 4096, 4096), (last + 1, 4096, 4096)], cus=cus)
        assert below[1] == 64 and at[1] != 64, (cus, below, at)


def test_thin_width_occupies_three_quarters_of_the_cus(sched):
    """The widest thin tile whose workgroups still occupy three quarters of the CUs (32 columns
    when none does)."""
    for M in (64, 100, 128, 192, 200, 256, 384, 512, 700, 1000, 1024):
        (_, bm, bn, _), = _plans(sched, [(M, 4096, 4096)])
        assert bm == 64
        wgs = lambda w: -(-M // 64) * -(-4096 // w)  # noqa: E731
        wider = [w for w in (128, 64, 32) if w > bn]
        assert bn == 32 or 4 * wgs(bn) >= 3 * CUS, (M, bn)
        assert all(4 * wgs(w) < 3 * CUS for w in wider), (M, bn)


def test_split_slices_fit_one_round_and_the_workspace(sched):
    for (M, N, K) in [(64, 256, 65536), (100, 512, 65536), (200, 512, 32768), (512, 256, 65536)]:
        (S, bm, bn, nbytes), = _plans(sched, [(M, N, K)])
        assert bn == 0 and S >= 2, (M, N, K)
        tiles = -(-M // bm) * -(-N // 256)
        assert S * tiles <= CUS and nbytes <= MAXB and S <= -(-K // 128)


FORCED = [
    # M, N, K, S, bm, bn -> S, bm, bn
    ((512, 4096, 4096, 0, 64, 128), (1, 64, 128)),   # thin with a chosen width
    ((512, 4096, 4096, 0, 64, 0), (1, 64, 128)),     # thin, automatic width
    ((512, 4096, 4096, 3, 64, 0), (1, 64, 128)),     # the thin kernel never splits
    ((512, 4096, 4096, 3, 0, 0), (3, 128, 0)),       # a forced split takes the fast kernel
    ((128, 4096, 4096, 0, 128, 0), (12, 128, 0)),    # 128-row tiles with their automatic split
    ((128, 4096, 4096, 1, 128, 0), (1, 128, 0)),     # ... and without a split
    ((1024, 4096, 4096, 0, 256, 0), (1, 256, 0)),    # 256-row tiles: M > 512, never split
    ((4096, 4096, 4096, 2, 0, 0), (2, 256, 0)),      # a split of the 256-row tiles
    ((512, 4096, 4096, 0, 0, 32), (1, 64, 32)),      # the automatic thin plan with a chosen width
    ((300, 520, 704, 100, 0, 0), (6, 128, 0)),       # S clamped to the 6 K-blocks
]


def test_forced_schedules(sched):
    got = sched([f"forced {M} {N} {K} {CUS} {S} {bm} {bn} {MAXB}" for (M, N, K, S, bm, bn), _ in FORCED])
    for (q, want), g in zip(FORCED, got):
        assert g[:3] == want, (q, g)


def test_forced_split_respects_the_workspace_bound(sched):
    (S, bm, bn, nbytes), = sched([f"forced 512 1024 8192 {CUS} 64 0 0 {MAXB}"])
    assert (S, bm, bn) == (64, 128, 0) and nbytes == 64 * 512 * 1024 * 4  # 128 MiB: over the 64 MiB scratch
    (S, _, _, nbytes), = sched([f"forced 512 1024 8192 {CUS} 64 0 0 {64 << 20}"])
    assert S == 32 and nbytes == 64 << 20


STAGES = [
    # bn, per_col, workgroups -> stages (160 KB of LDS per CU, 256 CUs)
    ((32, 0, 256), 12),     # 12.6 KB stages: twelve (151 KB) once per CU
    ((32, 0, 512), 6),      # six (75 KB) twice per CU
    ((32, 0, 768), 4),      # four (50 KB) three times per CU
    ((32, 0, 769), 3),
    ((64, 0, 256), 8),      # 16.7 KB stages: 133 KB, one per CU
    ((64, 0, 512), 4),      # 66.6 KB, two per CU
    ((64, 0, 513), 3),
    ((128, 0, 256), 6),     # 24.8 KB stages: 149 KB, one per CU
    ((128, 0, 512), 3),     # 74.5 KB, two per CU
    ((128, 0, 768), 2),     # 49.7 KB, three per CU
    ((128, 0, 5000), 2),    # more than one round at any depth: two
    ((128, 1, 512), 3),
]


def test_thin_pipeline_depth(sched):
    got = sched([f"stages {bn} {pc} {w} {CUS}" for (bn, pc, w), _ in STAGES])
    for (q, want), g in zip(STAGES, got):
        assert g[0] == want, (q, g)


# quantize_lhs row strips: (M, K) -> 16-byte pieces per thread
LHS_EXPECTED = {
    (4096, 4096): 8,      # 512 strips of 8 rows: two per CU, all resident
    (8192, 4096): 16,     # 512 strips of 16 rows
    (16384, 4096): 4,     # no size fits one round: 4
    (32768, 4096): 4,
    (2048, 4096): 4,      # 512 strips of 4 rows
    (1024, 4096): 2,
    (512, 4096): 1,       # 512 single rows
    (256, 4096): 1,       # fewer than two per CU even with one row each
    (2, 128): 1,
    (4096, 1280): 2,      # 10 K-blocks: 6-row strips of 2 pieces per thread, 683 of them
    (8192, 1280): 4,
    (4096, 7168): 8,      # two chunks of 28 K-blocks
    (4096, 14336): 4,     # four chunks of 28: more than one round at every size
}


def test_lhs_strip_sizes(sched):
    shapes = list(LHS_EXPECTED)
    got = sched([f"lhs {M} {(K + 127) // 128} {CUS}" for (M, K) in shapes])
    for sh, g in zip(shapes, got):
        assert g[0] == LHS_EXPECTED[sh], (sh, g)


def test_lhs_strip_size_is_always_launchable(sched):
    """Every answer is one of the instantiated sizes, for M from 1 to 65536 and K up to 32768."""
    qs = [f"lhs {M} {kb} {cus}" for M in (1, 7, 100, 513, 3000, 12345, 65536)
          for kb in (1, 2, 9, 32, 33, 100, 256) for cus in (256, 128, 80)]
    for g in sched(qs):
        assert g[0] in (1, 2, 4, 8, 16)


def test_header_is_self_contained(tmp_path):
    """schedule.hpp compiles on its own (nothing it needs comes from an earlier include)."""
    src = tmp_path / "only.cpp"
    src.write_text('#include "schedule.hpp"\nint main() { return bsfp8::sched::lhs_strip_loads(8192, 32, 256) == 16 ? 0 : 1; }\n')
    exe = str(tmp_path / "only")
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", exe], check=True)
    assert subprocess.run([exe]).returncode == 0


def test_thin_deepest_pipeline_fits_the_lds(sched):
    """The deepest instantiated thin pipeline per tile width: 12 stages of 64 x 32 tiles (12.3 KB
    each), 8 of 64 x 64 (16.3 KB), 6 of 64 x 128 (24.3 KB) within 160 KB, per-column scales too."""
    got = sched([f"maxstages {bn} {pc}" for bn in (32, 64, 128) for pc in (0, 1)])
    assert [g[0] for g in got] == [12, 12, 8, 8, 6, 6]


def test_thin_waves(sched):
    """8 waves (16-row waves) for 64- and 128-column thin tiles when the grid is at most one
    workgroup per CU (256 x 4096 x 4096 in 64 x 64 tiles: 13.9 us against 15.0 with 4 waves; 512
    rows in 64 x 128: 19.3 against 20.6-20.9), 4 otherwise (768 rows, 384 workgroups: 8 waves were
    slower) and always for 32-column tiles."""
    q = [(64, 256, 8), (128, 256, 8), (128, 200, 8), (64, 257, 4), (128, 384, 4), (32, 256, 4), (32, 100, 4)]
    got = sched([f"waves {bn} {w} {CUS}" for bn, w, _ in q])
    assert [g[0] for g in got] == [want for _, _, want in q]


# (M, N, K) -> (n1, S of the tail): a partial last round of 256 x 256 tiles runs its leading whole
# rounds of tile columns as one GEMM and the tail columns with K split
COLSPLIT = {
    (4096, 5120, 5120): (4096, 4),   # 320 tiles: 256 + 64 in 4 slices
    (4096, 5120, 4096): (4096, 4),
    (8192, 5120, 5120): (0, 1),      # 640 tiles: a tail of 128 would split only in 2 (measured slower)
    (4096, 5120, 2048): (0, 1),      # 16 K-blocks: the partial sums would cost more than they save
    (4096, 4096, 4096): (0, 1),      # whole rounds
    (16384, 5120, 5120): (0, 1),     # 1280 tiles: five whole rounds
    (6144, 4096, 4096): (0, 1),      # no whole-round prefix of tile columns (24 x nt1 never 256 k)
    (1024, 4096, 4096): (0, 1),      # the thin kernel's shape
}


def test_column_split(sched):
    shapes = list(COLSPLIT)
    got = sched([f"colsplit {M} {N} {K} {CUS} {MAXB}" for (M, N, K) in shapes])
    for sh, g in zip(shapes, got):
        assert (g[0], g[1] if g[0] else 1) == COLSPLIT[sh], (sh, g)
        if g[0]:
            M, N, K = sh
            assert g[0] % 256 == 0 and (-(-M // 256) * (g[0] // 256)) % CUS == 0
            assert g[2] == g[1] * M * ((N - g[0] + 7) // 8 * 8) * 4 <= MAXB
