"""GPU parity of the two scaled GEMMs against the CPU oracle.

The GEMMs run on the GPU's own codes and scales, which must first equal the oracle's bit for bit;
the oracle then evaluates the blockwise sum in fp64 on the same codes. Acceptance:
  max |C - C_o| <= 2e-2 (|C_o| + 1) elementwise and ||C - C_o||_F / ||C_o||_F <= 4e-3;
and for the end-to-end path SQNR against the fp64 matmul of the bf16 inputs >= 28 dB, within
0.05 dB of the oracle path's own SQNR.
Small problems are compared in full; full-size problems on a seeded sample of rows (always the
first and the last row, and any tail rows).
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests import _golden
from tests._gpu import DEV, to_dev

pytestmark = pytest.mark.gpu


def _cdiv(a, b):
    return (a + b - 1) // b


def _sample_rows(M, n=64, seed=0):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = set(g.choice(M, size=min(n, M), replace=False).tolist())
    rows |= {0, M - 1}
    rows |= set(range(M - M % 128, M))
    return np.array(sorted(rows), dtype=np.int64)


def _assert_close(c_gpu, c_or, what):
    rep = oracle.gemm_tolerance_report(c_gpu, c_or)
    assert rep["ok"], f"{what}: {rep}"
    return rep


def _codes(shape, seed, ld=None):
    """Random finite e4m3 codes [rows, cols] on the device, in a buffer with row stride ld."""
    g = np.random.Generator(np.random.PCG64(seed))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    h = g.choice(finite, size=shape)
    ld = ld or shape[1]
    buf = torch.zeros((shape[0], ld), dtype=torch.uint8, device=DEV)
    buf[:, :shape[1]] = torch.from_numpy(h).to(DEV)
    return h, buf[:, :shape[1]]


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.exp2(g.uniform(-10, 2, size=shape)).astype(np.float32)


GEMM_SHAPES = [
    # M, N, K, lda/ldb (multiple of 16), ldc
    (2, 512, 128, 128, 512), (130, 512, 1280, 1280, 512), (1, 1, 1, 16, 1), (3, 5, 300, 304, 5),
    (128, 128, 128, 128, 128), (129, 130, 129, 144, 131), (257, 384, 520, 528, 384),
    (64, 200, 4096, 4096, 200), (300, 260, 256, 256, 262),
    # 513 K-blocks, the last one partial: beyond the 128x128 fast path's staged B scales (general
    # kernel); the per-column variant stays on the fast path
    (40, 96, 65600, 65600, 96),
]


def _run_guarded(fn, M, N, ldc):
    cbuf = torch.full((M + 2, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    fn(cbuf[1:M + 1, :N])
    torch.cuda.synchronize()
    got = cbuf.float().cpu().numpy()
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[M + 1])), "write outside rows"
    assert np.all(np.isnan(got[1:M + 1, N:])), "write into row padding"
    return got[1:M + 1, :N]


def _quantized_operands(M, N, K, ld, seed, per_column):
    """A [M, K] and B [N, K] from seeded Gaussian bf16 data through the GPU quantizers (checked
    bit-exact against the oracle), padded to row stride ld. A ~ N(0,1) rows (1x128 scales);
    B ~ N(0, 0.02^2) as a weight (128x128 scales) or as 128x1 column groups of a [K, N] tensor."""
    g = np.random.Generator(np.random.PCG64(seed))
    ah = inputs.bf16_bits_from_f64(g.standard_normal((M, K)))
    qa = torch.zeros((M, ld), dtype=torch.uint8, device=DEV)[:, :K]
    qa, sa = bf.quantize_lhs(to_dev(ah), q=qa)
    oqa, osa = oracle.quantize_lhs(ah)
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(sa.cpu().numpy(), osa)
    if per_column:
        xh = inputs.bf16_bits_from_f64(g.standard_normal((K, N)) * 0.02)   # [K, N], groups down K
        qb = torch.zeros((N, ld), dtype=torch.uint8, device=DEV)[:, :K]
        qb, sb = bf.quantize_rhs(to_dev(xh), qT=qb)
        oqb, osb = oracle.quantize_rhs(xh)
    else:
        wh = inputs.bf16_bits_from_f64(g.standard_normal((N, K)) * 0.02)
        qb = torch.zeros((N, ld), dtype=torch.uint8, device=DEV)[:, :K]
        qb, _, sb = bf.quantize_weight_128x128(to_dev(wh), q=qb, want_qT=False)
        oqb, _, osb = oracle.quantize_weight_128x128(wh, want_qT=False)
    assert np.array_equal(qb.cpu().numpy(), oqb) and np.array_equal(sb.cpu().numpy(), osb)
    return qa, sa, qb, sb, oqa, osa, oqb, osb


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x128_ragged(M, N, K, ld, ldc):
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, ld, M + N + K, False)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x128(qa, sa, qb, sb, c=c), M, N, ldc)
    co = oracle.gemm_1x128_128x128(oqa, osa, oqb, osb, osb.shape[1], 1)
    _assert_close(got, co, "gemm_1x128_128x128")


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x1_ragged(M, N, K, ld, ldc):
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, ld, M + N + K + 1, True)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x1(qa, sa, qb, sb, c=c), M, N, ldc)
    co = oracle.gemm_1x128_128x1(oqa, osa, oqb, osb)
    _assert_close(got, co, "gemm_1x128_128x1")


def _abs_codes(h):
    return h & 0x7F


def _assert_dot_bound(got, co, c_abs, what):
    """Full-range random codes: the matrix core's 128-term fp8 dot product is not an exactly
    rounded fp32 sum (its error reaches about 2^-12 of the sum of |products|), so under heavy
    cancellation the error is bounded by the absolute-value sum, not by |C|. Bound used:
    |C - C_o| <= 2^-10 * sum_kb |f_kb| sum_k |a_k b_k|  +  2^-8 |C_o|  (bf16 output rounding)."""
    bound = 2.0 ** -10 * c_abs + 2.0 ** -8 * np.abs(co)
    excess = np.abs(got - co) - bound
    assert np.all(excess <= 0), f"{what}: {int(np.count_nonzero(excess > 0))} elements over bound"
    nf = np.linalg.norm(co)
    assert np.linalg.norm(got - co) <= 4e-3 * nf, f"{what}: relative Frobenius"


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x128_full_range_codes(M, N, K, ld, ldc):
    Kb, Nb = _cdiv(K, 128), _cdiv(N, 128)
    ah, a = _codes((M, K), 1, ld)
    bh, b = _codes((N, K), 2, ld)
    a_s, b_s = _scales((Kb, M), 3), _scales((Nb, Kb), 4)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x128(a, to_dev(a_s), b, to_dev(b_s), Kb, 1, c=c),
                       M, N, ldc)
    co = oracle.gemm_1x128_128x128(ah, a_s, bh, b_s, Kb, 1)
    c_abs = oracle.gemm_1x128_128x128(_abs_codes(ah), a_s, _abs_codes(bh), b_s, Kb, 1)
    _assert_dot_bound(got, co, c_abs, "gemm_1x128_128x128")


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x1_full_range_codes(M, N, K, ld, ldc):
    Kb = _cdiv(K, 128)
    ah, a = _codes((M, K), 5, ld)
    bh, b = _codes((N, K), 6, ld)
    a_s, b_s = _scales((Kb, M), 7), _scales((Kb, N), 8)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x1(a, to_dev(a_s), b, to_dev(b_s), c=c), M, N, ldc)
    co = oracle.gemm_1x128_128x1(ah, a_s, bh, b_s)
    c_abs = oracle.gemm_1x128_128x1(_abs_codes(ah), a_s, _abs_codes(bh), b_s)
    _assert_dot_bound(got, co, c_abs, "gemm_1x128_128x1")


def test_gemm_transposed_scale_strides():
    """dgrad reads the weight's [Nb_w, Kb_w] scales transposed through the strides."""
    M, N, K = 256, 384, 512
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, K, 11, False)
    sbt = np.ascontiguousarray(osb.T)          # stored [Kb, Nb]: element (kb, nb) at kb * Nb + nb
    Nb = sbt.shape[1]
    c = bf.gemm_1x128_128x128(qa, sa, qb, to_dev(sbt), 1, Nb)
    co = oracle.gemm_1x128_128x128(oqa, osa, oqb, sbt, 1, Nb)
    _assert_close(c.float().cpu().numpy(), co, "strided b_s")


def test_gemm_k_zero_writes_zeros():
    M, N = 5, 40
    c = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((M, 16), dtype=torch.uint8, device=DEV)[:, :0]
    b = torch.zeros((N, 16), dtype=torch.uint8, device=DEV)[:, :0]
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    bf.gemm_1x128_128x128(a, one, b, one, 1, 1, c=c, K=0)
    torch.cuda.synchronize()
    assert torch.all(c == 0)


# ------------------------------------------------------------------ end-to-end on the workloads

def _forward_check(a_h, w_h, rows, sqnr_min=28.0):
    a, w = to_dev(a_h), to_dev(w_h)
    qa, sa = bf.quantize_lhs(a)
    qw, _, sw = bf.quantize_weight_128x128(w, want_qT=False)
    c = bf.gemm_1x128_128x128(qa, sa, qw, sw)
    torch.cuda.synchronize()
    oqa, osa = oracle.quantize_lhs(a_h)
    oqw, _, osw = oracle.quantize_weight_128x128(w_h, want_qT=False)
    qa_h, sa_h = qa.cpu().numpy(), sa.cpu().numpy()
    assert np.array_equal(qa_h, oqa) and np.array_equal(sa_h, osa)
    assert np.array_equal(qw.cpu().numpy(), oqw) and np.array_equal(sw.cpu().numpy(), osw)
    co = oracle.gemm_1x128_128x128(oqa, osa, oqw, osw, osw.shape[1], 1, rows=rows)
    cg = c.float().cpu().numpy()[rows]
    _assert_close(cg, co, "forward")
    ref = oracle.matmul_bf16_f64(a_h, w_h, rows=rows)
    s_gpu, s_or = oracle.sqnr_db(ref, cg), oracle.sqnr_db(ref, co)
    assert s_gpu >= sqnr_min, (s_gpu, s_or)
    assert abs(s_gpu - s_or) <= 0.05, (s_gpu, s_or)
    return s_gpu, s_or


@pytest.mark.parametrize("idx", [0, 1])
def test_forward_small_workloads_full(idx):
    d = inputs.make_workload(idx)
    M = d["A"].shape[0]
    _forward_check(d["A"], d["W"], np.arange(M), sqnr_min=28.0)


@pytest.mark.parametrize("row", _golden.table("pages_sqnr_table.txt"),
                         ids=lambda r: "x".join(str(int(v)) for v in r[:3]))
def test_sqnr_at_pages_table_shapes(row):
    """The GPU path at every shape of the ROCm page's GEMM-correctness table (SQNR 28.6-28.8 dB
    against a BF16 matmul): at least 28 dB, within the table's band of the printed value (1.2 dB
    for the tiny M = 2, 4 outputs, 0.3 dB otherwise, as for the oracle path) and within 0.05 dB of
    the oracle path on the same inputs (A ~ N(0,1), W ~ N(0, 0.02^2), seed 0)."""
    M, N, K, db = int(row[0]), int(row[1]), int(row[2]), row[3]
    g = inputs.rng(0)
    a_h = inputs.normal_bf16(g, (M, K))
    w_h = inputs.normal_bf16(g, (N, K), 0.02)
    rows = np.arange(M) if M <= 128 else np.linspace(0, M - 1, 64).astype(np.int64)
    band = 1.2 if M * N < 100000 else 0.3
    s_gpu, _ = _forward_check(a_h, w_h, rows, sqnr_min=max(28.0, db - band))  # never below 28 dB
    assert abs(s_gpu - db) <= band, s_gpu


def test_forward_4096_full():
    """All 4096 x 4096 outputs of the 4096^3 forward against the oracle."""
    d = inputs.make_workload(2)
    _forward_check(d["A"], d["W"], np.arange(4096))


def test_forward_outlier_sampled():
    """16384 x 5120 x 5120 with outlier channels and 1% zero elements: 512 seeded rows plus the
    first and last."""
    d = inputs.make_workload(4)
    _forward_check(d["A"], d["W"], _sample_rows(16384, 512))


def test_forward_outlier_zero_groups_sampled():
    """The same shape with 1% of whole 1x128 groups zero (their scale is the eps clamp's)."""
    d = inputs.make_workload(4, zero_groups=True)
    _forward_check(d["A"], d["W"], _sample_rows(16384, 256, seed=1))


def test_training_step_full_size_sampled():
    """Forward Y = X W^T, dgrad dX = dY W (transposed weight codes, transposed scale strides) and
    wgrad dW = dY^T X (128x1 scales, contracting over the 8192 tokens)."""
    d = inputs.make_workload(3)
    Xh, Wh, dYh = d["X"], d["W"], d["dY"]
    X, W, dY = to_dev(Xh), to_dev(Wh), to_dev(dYh)
    qx, sx = bf.quantize_lhs(X)
    qdy, sdy = bf.quantize_lhs(dY)
    qxT, sxT = bf.quantize_rhs(X)
    qdyT, sdyT = bf.quantize_rhs(dY)
    qw, qwT, sw = bf.quantize_weight_128x128(W)
    Kbw = sw.shape[1]
    y = bf.gemm_1x128_128x128(qx, sx, qw, sw)                      # [8192, 4096]
    dx = bf.gemm_1x128_128x128(qdy, sdy, qwT, sw, 1, Kbw)          # [8192, 4096]
    dw = bf.gemm_1x128_128x1(qdyT, sdyT, qxT, sxT)                 # [4096, 4096]
    torch.cuda.synchronize()

    o = {}
    o["qx"], o["sx"] = oracle.quantize_lhs(Xh)
    o["qdy"], o["sdy"] = oracle.quantize_lhs(dYh)
    o["qxT"], o["sxT"] = oracle.quantize_rhs(Xh)
    o["qdyT"], o["sdyT"] = oracle.quantize_rhs(dYh)
    o["qw"], o["qwT"], o["sw"] = oracle.quantize_weight_128x128(Wh)
    for name, t in [("qx", qx), ("sx", sx), ("qdy", qdy), ("sdy", sdy), ("qxT", qxT),
                    ("sxT", sxT), ("qdyT", qdyT), ("sdyT", sdyT), ("qw", qw), ("qwT", qwT),
                    ("sw", sw)]:
        assert np.array_equal(t.cpu().numpy(), o[name]), name

    rows = _sample_rows(8192, 512)
    co = oracle.gemm_1x128_128x128(o["qx"], o["sx"], o["qw"], o["sw"], Kbw, 1, rows=rows)
    _assert_close(y.float().cpu().numpy()[rows], co, "forward")
    co = oracle.gemm_1x128_128x128(o["qdy"], o["sdy"], o["qwT"], o["sw"], 1, Kbw, rows=rows)
    _assert_close(dx.float().cpu().numpy()[rows], co, "dgrad")
    rows_w = _sample_rows(4096, 512)
    co = oracle.gemm_1x128_128x1(o["qdyT"], o["sdyT"], o["qxT"], o["sxT"], rows=rows_w)
    _assert_close(dw.float().cpu().numpy()[rows_w], co, "wgrad")
    # SQNR of each product against the fp64 matmul of the bf16 operands
    xf = oracle.bf16_bits_to_f64(Xh)
    dyf = oracle.bf16_bits_to_f64(dYh)
    wf = oracle.bf16_bits_to_f64(Wh)
    ref_dx = dyf[rows] @ wf
    ref_dw = dyf.T[rows_w] @ xf
    assert oracle.sqnr_db(ref_dx, dx.float().cpu().numpy()[rows]) >= 28.0
    assert oracle.sqnr_db(ref_dw, dw.float().cpu().numpy()[rows_w]) >= 28.0


@pytest.mark.parametrize("per_col", [False, True], ids=["128x128", "128x1"])
@pytest.mark.parametrize("M,N,K,ld", [(300, 260, 200, 208), (257, 384, 1000, 1008), (64, 128, 1, 16),
                                      (130, 512, 1280 - 40, 1248)], ids=lambda v: str(v))
def test_gemm_partial_last_block_ignores_nan_padding(M, N, K, ld, per_col):
    """A partial last K-block: the bytes at and past K of every operand row (row padding, and for
    the last row the next allocation) hold the NaN code 0x7F; none of it may reach C."""
    g = np.random.Generator(np.random.PCG64(M + K))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ah = g.choice(finite, size=(M, K))
    bh = g.choice(finite, size=(N, K))
    Kb = _cdiv(K, 128)

    def nan_padded(h):
        buf = torch.full((h.shape[0] + 1, ld), 0x7F, dtype=torch.uint8, device=DEV)
        buf[:h.shape[0], :K] = torch.from_numpy(h).to(DEV)
        return buf[:h.shape[0], :K]

    a, b = nan_padded(ah), nan_padded(bh)
    a_s = _scales((Kb, M), 21)
    if per_col:
        b_s = _scales((Kb, N), 22)
        got = _run_guarded(lambda c: bf.gemm_1x128_128x1(a, to_dev(a_s), b, to_dev(b_s), c=c), M, N, N)
        co = oracle.gemm_1x128_128x1(ah, a_s, bh, b_s)
        c_abs = oracle.gemm_1x128_128x1(_abs_codes(ah), a_s, _abs_codes(bh), b_s)
    else:
        b_s = _scales((_cdiv(N, 128), Kb), 23)
        got = _run_guarded(lambda c: bf.gemm_1x128_128x128(a, to_dev(a_s), b, to_dev(b_s), Kb, 1, c=c),
                           M, N, N)
        co = oracle.gemm_1x128_128x128(ah, a_s, bh, b_s, Kb, 1)
        c_abs = oracle.gemm_1x128_128x128(_abs_codes(ah), a_s, _abs_codes(bh), b_s, Kb, 1)
    assert np.all(np.isfinite(got))
    _assert_dot_bound(got, co, c_abs, "partial last K-block")


# ------------------------------------------------------------------ the split-K path

SPLIT_SHAPES = [
    # M, N, K, ld: ragged tiles, a partial last K-block, one tile, several tiles
    (130, 300, 1000, 1008), (1, 40, 4096, 4096), (257, 513, 2000, 2000), (64, 256, 384, 384),
    (300, 260, 200, 208),
]


@pytest.mark.parametrize("per_col", [False, True], ids=["128x128", "128x1"])
@pytest.mark.parametrize("bm", [256, 128], ids=["tile256", "tile128"])
@pytest.mark.parametrize("S", [1, 2, 3, 7])
@pytest.mark.parametrize("M,N,K,ld", SPLIT_SHAPES, ids=lambda v: str(v))
def test_gemm_forced_schedule(M, N, K, ld, S, bm, per_col, monkeypatch):
    """Every schedule on ragged shapes: tile height bm (BSFP8_GEMM_TILE_M) and K split over S
    slices (BSFP8_GEMM_SPLIT; 1 = none): fp32 partial tiles summed by the second kernel, against the
    oracle in full; the fixed summation order makes two calls agree bit for bit."""
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, ld, M + N + K + S, per_col)
    monkeypatch.setenv("BSFP8_GEMM_SPLIT", str(S))
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", str(bm))
    if per_col:
        fn = lambda c: bf.gemm_1x128_128x1(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x1(oqa, osa, oqb, osb)
    else:
        fn = lambda c: bf.gemm_1x128_128x128(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x128(oqa, osa, oqb, osb, osb.shape[1], 1)
    got = _run_guarded(fn, M, N, N + 3)
    again = _run_guarded(fn, M, N, N + 3)
    assert np.array_equal(got, again)
    _assert_close(got, co, f"split {S}")


THIN_SHAPES = SPLIT_SHAPES + [
    # one row; M at and around the 64-row tile; a column tail inside a 4-column group; K < 128
    (1, 4100, 640, 640), (64, 96, 256, 256), (65, 130, 384, 400), (127, 33, 100, 112), (2, 512, 128, 128),
]


@pytest.mark.parametrize("per_col", [False, True], ids=["128x128", "128x1"])
@pytest.mark.parametrize("bn", [32, 64, 128], ids=lambda v: f"bn{v}")
@pytest.mark.parametrize("M,N,K,ld", THIN_SHAPES, ids=lambda v: str(v))
def test_gemm_thin_schedule(M, N, K, ld, bn, per_col, monkeypatch):
    """The thin kernel (BSFP8_GEMM_TILE_M=64, tile width BSFP8_GEMM_TILE_N) on ragged shapes:
    against the oracle in full, and bit for bit against the fast kernel's 128-row tiles (8 waves of
    32 rows) and 256-row tiles (8 waves of 64 rows) without a split: the three apply the same
    per-K-block arithmetic to every output in the same order."""
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, ld, M + 3 * N + K + bn, per_col)
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    if per_col:
        fn = lambda c: bf.gemm_1x128_128x1(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x1(oqa, osa, oqb, osb)
    else:
        fn = lambda c: bf.gemm_1x128_128x128(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x128(oqa, osa, oqb, osb, osb.shape[1], 1)
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", "64")
    monkeypatch.setenv("BSFP8_GEMM_TILE_N", str(bn))
    got = _run_guarded(fn, M, N, N + 3)
    _assert_close(got, co, f"thin {bn}")
    monkeypatch.setenv("BSFP8_GEMM_SPLIT", "1")
    monkeypatch.delenv("BSFP8_GEMM_TILE_N")
    for bm in (128, 256):
        monkeypatch.setenv("BSFP8_GEMM_TILE_M", str(bm))
        fast = _run_guarded(fn, M, N, N + 3)
        assert np.array_equal(got.view(np.uint32), fast.view(np.uint32)), f"thin and {bm}-row tiles differ"


# K-block counts 1, 2, 3 (one pair and a single), 5 and 16; partial last blocks (K = 200, 650,
# 4000); the depths each tile width instantiates (2 and 3: one block per barrier; 4 and more: two)
STAGE_SHAPES = [(70, 200, 128, 128), (65, 136, 200, 208), (130, 100, 384, 384), (70, 260, 650, 656),
                (129, 520, 2048, 2048), (70, 4096, 4000, 4000)]
STAGES_OF = {32: (2, 3, 4, 6, 8, 12), 64: (2, 3, 4, 6, 8), 128: (2, 3, 4, 6)}


@pytest.mark.parametrize("per_col", [False, True], ids=["128x128", "128x1"])
@pytest.mark.parametrize("bn", [32, 64, 128], ids=lambda v: f"bn{v}")
@pytest.mark.parametrize("M,N,K,ld", STAGE_SHAPES, ids=lambda v: str(v))
def test_gemm_thin_every_pipeline_depth(M, N, K, ld, bn, per_col, monkeypatch):
    """Every LDS pipeline depth of the thin kernel (BSFP8_GEMM_THIN_STAGES), with 4 and (64- and
    128-column tiles) 8 waves per workgroup (BSFP8_GEMM_THIN_WAVES), gives the same bits as the fast
    kernel's 128-row tiles without a split, and the oracle's values; a depth the tile's LDS cannot
    hold, or a wave count the width has no layout for, is refused."""
    qa, sa, qb, sb, oqa, osa, oqb, osb = _quantized_operands(M, N, K, ld, M + 5 * N + K + bn, per_col)
    if per_col:
        fn = lambda c: bf.gemm_1x128_128x1(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x1(oqa, osa, oqb, osb)
    else:
        fn = lambda c: bf.gemm_1x128_128x128(qa, sa, qb, sb, c=c)
        co = oracle.gemm_1x128_128x128(oqa, osa, oqb, osb, osb.shape[1], 1)
    monkeypatch.setenv("BSFP8_GEMM_SPLIT", "1")
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", "128")
    ref = _run_guarded(fn, M, N, N + 3)
    _assert_close(ref, co, "128-row tiles")
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", "64")
    monkeypatch.setenv("BSFP8_GEMM_TILE_N", str(bn))
    for waves in ((4, 8) if bn >= 64 else (4,)):
        monkeypatch.setenv("BSFP8_GEMM_THIN_WAVES", str(waves))
        for st in STAGES_OF[bn]:
            monkeypatch.setenv("BSFP8_GEMM_THIN_STAGES", str(st))
            got = _run_guarded(fn, M, N, N + 3)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{waves} waves, {st} stages"
    monkeypatch.setenv("BSFP8_GEMM_THIN_STAGES", str(max(STAGES_OF[bn]) * 2))
    with pytest.raises(bf.Bsfp8Error):
        fn(torch.empty((M, N), dtype=torch.bfloat16, device=DEV))
    monkeypatch.delenv("BSFP8_GEMM_THIN_STAGES")
    monkeypatch.setenv("BSFP8_GEMM_THIN_WAVES", "8" if bn == 32 else "6")  # not a layout of this width
    with pytest.raises(bf.Bsfp8Error):
        fn(torch.empty((M, N), dtype=torch.bfloat16, device=DEV))


def test_gemm_column_split(monkeypatch):
    """4096 x 5120 x 4096 (320 tiles of 256 x 256: one round and a quarter) runs its first 4096
    columns as one GEMM and the last 1024 with K split in 4: the leading columns equal the unsplit
    schedule bit for bit (same tiles, same order), every column is within the oracle's tolerance on
    sampled rows, and the allocation-free entry point (its tail slices in the static scratch) gives
    the same bits."""
    M, N, K = 4096, 5120, 4096
    g = inputs.rng(11)
    a_h = inputs.normal_bf16(g, (M, K))
    w_h = inputs.normal_bf16(g, (N, K), 0.02)
    oqa, osa = oracle.quantize_lhs(a_h)
    oqw, _, osw = oracle.quantize_weight_128x128(w_h, want_qT=False)
    qa, sa, qw, sw = to_dev(oqa), to_dev(osa), to_dev(oqw), to_dev(osw)
    for k in ("BSFP8_GEMM_SPLIT", "BSFP8_GEMM_TILE_M", "BSFP8_GEMM_TILE_N", "BSFP8_GEMM_COLUMN_SPLIT"):
        monkeypatch.delenv(k, raising=False)
    split = bf.gemm_1x128_128x128(qa, sa, qw, sw).cpu().float().numpy()
    c_na = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    bf.gemm_1x128_128x128_noalloc(qa, sa, qw, sw, c_na)
    assert np.array_equal(c_na.cpu().float().numpy().view(np.uint32), split.view(np.uint32))
    monkeypatch.setenv("BSFP8_GEMM_COLUMN_SPLIT", "0")
    whole = bf.gemm_1x128_128x128(qa, sa, qw, sw).cpu().float().numpy()
    assert np.array_equal(split[:, :4096].view(np.uint32), whole[:, :4096].view(np.uint32))
    rows = _sample_rows(M, 256, seed=5)
    co = oracle.gemm_1x128_128x128(oqa, osa, oqw, osw, osw.shape[1], 1, rows=rows)
    _assert_close(split[rows], co, "column split")


@pytest.mark.parametrize("M,N,K", [(128, 4096, 4096), (512, 4096, 4096), (2048, 4096, 4096),
                                   (2, 5120, 1280), (4, 3584, 640)], ids=lambda v: str(v))
def test_forward_short_wide_shapes_full(M, N, K, monkeypatch):
    """The pages' short-and-wide GEMM shapes, which the automatic plan gives to the thin kernel
    (2048 rows: the fast kernel's 128-row tiles): every output row against the oracle, and the SQNR
    against the fp64 matmul of the bf16 inputs."""
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    monkeypatch.delenv("BSFP8_GEMM_TILE_M", raising=False)
    monkeypatch.delenv("BSFP8_GEMM_TILE_N", raising=False)
    g = inputs.rng(0)
    a_h = inputs.normal_bf16(g, (M, K))
    w_h = inputs.normal_bf16(g, (N, K), 0.02)
    _forward_check(a_h, w_h, np.arange(M), sqnr_min=28.0)  # the oracle path: 28.66-28.74 dB here


@pytest.mark.parametrize("bm", [256, 128, 64], ids=["tile256", "tile128", "thin"])
def test_gemm_operand_row_stride_at_the_limit(bm, monkeypatch):
    """Operand rows 2^23 bytes apart, the largest stride the GEMMs accept (256 rows of a tile then
    span exactly 2^31 bytes, the size of a buffer resource): ragged M and N against the oracle."""
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", str(bm))
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    M, N, K, ld = 200, 300, 256, 2 ** 23
    g = np.random.Generator(np.random.PCG64(62))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ah, bh = g.choice(finite, size=(M, K)), g.choice(finite, size=(N, K))
    a = torch.zeros((M, ld), dtype=torch.uint8, device=DEV)
    b = torch.zeros((N, ld), dtype=torch.uint8, device=DEV)
    a[:, :K] = torch.from_numpy(ah).to(DEV)
    b[:, :K] = torch.from_numpy(bh).to(DEV)
    Kb = _cdiv(K, 128)
    a_s, b_s = _scales((Kb, M), 63), _scales((_cdiv(N, 128), Kb), 64)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x128(a[:, :K], to_dev(a_s), b[:, :K], to_dev(b_s), Kb, 1, c=c),
                       M, N, N)
    co = oracle.gemm_1x128_128x128(ah, a_s, bh, b_s, Kb, 1)
    c_abs = oracle.gemm_1x128_128x128(_abs_codes(ah), a_s, _abs_codes(bh), b_s, Kb, 1)
    _assert_dot_bound(got, co, c_abs, "row stride 2^23")
    del a, b
    torch.cuda.empty_cache()


def test_split_gemms_on_two_streams_concurrently(monkeypatch):
    """The split-K workspace comes from a stream-ordered pool: split GEMMs enqueued on two streams
    at once get separate workspaces, and every result equals the same call made alone. (128-row
    tiles forced: these shapes would otherwise take the thin kernel, which does not split.)"""
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    monkeypatch.setenv("BSFP8_GEMM_TILE_M", "128")
    monkeypatch.delenv("BSFP8_GEMM_TILE_N", raising=False)
    shapes = [(128, 4096, 4096), (64, 2048, 3072)]
    ops, ref = [], []
    for i, (M, N, K) in enumerate(shapes):
        qa, sa, qb, sb, *_ = _quantized_operands(M, N, K, K, 70 + i, False)
        ops.append((qa, sa, qb, sb))
        ref.append(bf.gemm_1x128_128x128(qa, sa, qb, sb))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(r) for _ in range(6)] for r in ref]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(6):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                bf.gemm_1x128_128x128(*ops[i], c=outs[i][rep], stream=s)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        for rep in range(6):
            assert torch.equal(outs[i][rep].view(torch.int16), ref[i].view(torch.int16)), (i, rep)
