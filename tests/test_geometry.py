"""CPU check of the kernels' index arithmetic (csrc/geometry.hpp, the header the GEMM kernels and
quantize_lhs call), compiled with the host compiler and enumerated lane by lane by
tests/geometry_check.cpp -- the device-free test of "Mask a_s/b_s scale loads in blockwise FP8
training GEMM kernels" (Test: masked scale indices never leave [0, M) / [0, N) and cover every valid
row and column), extended to every operand and scale read, every output store and the LHS
quantizer's column-major scale stores (root-cause comment of "Enable blockwise FP8 dense training
kernels on ROCm").

Planted mistakes -- the pages' two bugs, an A-scale read without the row mask and a scale store
without the row mask (in the tile and in the row-strip LHS quantizer), and lane masks of the GEMM
kernels -- are compiled into scratch copies of the header and must make the check fail.
"""
import itertools
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_act_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "geometry_check.cpp")

# the sizes named for this check: around one and two tiles, the 128-group edge, and past 4096
SIZES = [1, 2, 127, 128, 129, 130, 255, 256, 257, 4097]


def _build(tmp_path, header_dir=CSRC, name="geometry_check"):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I", header_dir, SRC, "-o", exe], check=True)
    return exe


def _run(exe, shapes):
    args = [str(v) for s in shapes for v in s]
    return subprocess.run([exe, *args], capture_output=True, text=True)


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    return _build(tmp_path_factory.mktemp("geom"))


def test_every_shape_of_the_grid(checker):
    """All M, N, K in SIZES (1000 shapes, K-blocks, ragged tiles, partial K-blocks)."""
    shapes = list(itertools.product(SIZES, SIZES, SIZES))
    for i in range(0, len(shapes), 100):
        r = _run(checker, shapes[i:i + 100])
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        assert r.stdout.count("ok M=") == len(shapes[i:i + 100])


def test_workload_shapes(checker):
    """The workloads' GEMM shapes (forward, dgrad, wgrad over the tokens, the pages' table)."""
    shapes = [(2, 512, 128), (130, 5120, 1280), (4096, 4096, 4096), (8192, 4096, 4096),
              (4096, 4096, 8192), (128, 4096, 4096), (512, 4096, 4096), (2, 5120, 1280),
              (4, 3584, 640), (4096, 8192, 4096), (4096, 5120, 5120)]
    r = _run(checker, shapes)
    assert r.returncode == 0, r.stdout[-2000:]


def test_lhs_strip_shapes(checker):
    """quantize_lhs's row strips: K with a partial last group (144, 4112), K split into chunks of
    K-blocks (5248 = 41 blocks in chunks of 21 and 20, 8192, 12304), ragged strips of rows."""
    shapes = [(130, 1, 144), (1, 1, 16), (257, 1, 4112), (4097, 1, 5248), (8192, 1, 8192),
              (4096, 1, 4096), (2, 1, 1280), (3, 1, 640), (1000, 1, 12304)]
    r = _run(checker, shapes)
    assert r.returncode == 0, r.stdout[-2000:]


def _planted(tmp_path, old, new, name):
    d = tmp_path / name
    d.mkdir()
    src = open(os.path.join(CSRC, "geometry.hpp")).read()
    assert src.count(old) == 1
    (d / "geometry.hpp").write_text(src.replace(old, new))
    return _build(tmp_path, str(d), name + "_check")


def test_unmasked_scale_read_is_caught(tmp_path):
    """The bug of the masking page: the A-scale read of rows >= M left unmasked."""
    exe = _planted(tmp_path,
                   "return (lane < rows_per_wave && m < m_end) ? static_cast<uint32_t>(4 * m) : kOob;",
                   "return lane < rows_per_wave ? static_cast<uint32_t>(4 * m) : kOob;", "planted_read")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "a_s row" in r.stdout, r.stdout


def test_unmasked_scale_store_is_caught(tmp_path):
    """The bug of the root-cause comment: LHS scale stores of rows >= M (they alias column kb + 1)."""
    exe = _planted(tmp_path, "BSFP8_HD bool row_stored(int64_t m, int64_t M) { return m < M; }",
                   "BSFP8_HD bool row_stored(int64_t m, int64_t M) { return m < M + 64; }", "planted_store")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "a_s store" in r.stdout, r.stdout


def test_unmasked_strip_scale_store_is_caught(tmp_path):
    """The root-cause comment's bug in the row-strip kernel: scale stores of rows >= M."""
    exe = _planted(tmp_path, "return i < s.rows * s.g && m < M && kb < Kb;",
                   "return i < s.rows * s.g && kb < Kb;", "planted_strip")
    r = _run(exe, [(130, 1, 256)])
    assert r.returncode != 0 and "strip a_s store" in r.stdout, r.stdout


def test_planted_thin_pipeline_short_wait_is_caught(tmp_path):
    """The thin kernel's wait letting one block too many stay in flight: a block is multiplied
    before its loads have landed."""
    exe = _planted(tmp_path, "const int a = thin_ahead(stages) - n, b = Kb - kb - n;",
                   "const int a = thin_ahead(stages) - n + 1, b = Kb - kb - n + 1;", "planted_wait")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "before its loads landed" in r.stdout, r.stdout


def test_planted_thin_pipeline_stage_overrun_is_caught(tmp_path):
    """Issuing one block further ahead than the stages allow overwrites a stage still in use."""
    exe = _planted(tmp_path, "BSFP8_HD constexpr int thin_ahead(int stages) { return stages - thin_blocks_per_step(stages); }",
                   "BSFP8_HD constexpr int thin_ahead(int stages) { return stages - thin_blocks_per_step(stages) + 1; }",
                   "planted_ahead")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "still holding" in r.stdout, r.stdout


def test_planted_operand_row_read_is_caught(tmp_path):
    """An operand resource that runs past the tile's in-range rows."""
    exe = _planted(tmp_path,
                   "return rows_in_range > 8 * (q & 3) ? (rows_in_range - 8 * (q & 3)) * ld : 0;",
                   "return (256 - 8 * (q & 3)) * ld;", "planted_rows")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0, r.stdout


def test_planted_thin_scale_read_is_caught(tmp_path):
    """The masking page's bug in the thin kernel: its A-scale read of rows >= M left unmasked."""
    exe = _planted(tmp_path,
                   "return m0 + lane < M ? static_cast<uint32_t>(4 * (m0 + lane)) : kOob;",
                   "return static_cast<uint32_t>(4 * (m0 + lane));", "planted_thin_read")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "thin a_s row" in r.stdout, r.stdout


def test_planted_thin_bscale_lane_is_caught(tmp_path):
    """A per-column B-scale load of the thin kernel whose lanes run past the tile's columns."""
    exe = _planted(tmp_path,
                   "return !per_col ? 1ull : (bn >= 64 ? ~0ull : ((1ull << bn) - 1));",
                   "return !per_col ? 1ull : ~0ull;", "planted_thin_bs")
    r = _run(exe, [(130, 256, 256)])
    assert r.returncode != 0 and "outside the tile" in r.stdout, r.stdout


def test_checker_needs_no_hip():
    """The header compiles for the host with the plain C++ compiler (no HIP headers)."""
    assert shutil.which("g++") is not None
    src = open(os.path.join(CSRC, "geometry.hpp")).read()
    assert "hip_runtime" not in src
