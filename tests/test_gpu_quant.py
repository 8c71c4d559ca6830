"""GPU parity of the three quantizers and the element conversion against the CPU oracle.

Codes and scales must match bit for bit. Outputs are guard-banded views (sentinel bytes around and
between rows, NaN-prefilled scales) so a stray store, such as a scale row >= M landing in the next
K-block column of the column-major layout, fails the test.
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests import _golden
from tests._gpu import DEV, GuardedF32, GuardedU8, bf16_view, to_dev

pytestmark = pytest.mark.gpu


def _cdiv(a, b):
    return (a + b - 1) // b


def _rand_bf16(shape, seed, spread=True):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape)
    if spread:
        x *= np.exp2(g.integers(-20, 20, size=(shape[0], 1)))
    return inputs.bf16_bits_from_f64(x)


# ------------------------------------------------------------------ element conversion

@pytest.mark.parametrize("chunk", range(16))
def test_encode_exhaustive_vs_oracle(chunk):
    """Every binary32 bit pattern (16 chunks of 2^28): device conversion == oracle encoder.
    NaN patterns are outside the contract and skipped."""
    n = 1 << 28
    first = chunk * n
    idx = torch.arange(first, first + n, dtype=torch.int64, device=DEV)
    idx = torch.where(idx >= 2 ** 31, idx - 2 ** 32, idx).to(torch.int32)
    x = idx.view(torch.float32)
    q = bf.encode_e4m3_f32(x)
    got = q.cpu().numpy()
    del idx, x, q
    ref = oracle.e4m3_encode_bits(first, n)
    bits = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32)
    nan = (bits & 0x7F800000) == 0x7F800000
    nan &= (bits & 0x007FFFFF) != 0
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, (f"{bad.size} mismatches; first at bits {hex(first + int(bad[0]))}: "
                           f"gpu {got[bad[0]]:#x} oracle {ref[bad[0]]:#x}")


# ------------------------------------------------------------------ quantize_lhs

LHS_SHAPES = [
    (2, 128, 128, 128),        # small forward case
    (130, 1280, 1280, 1280),   # M tail: rows 128, 129 of the second 64-row tile
    (1, 1, 1, 1), (3, 127, 128, 127), (7, 129, 136, 129), (5, 200, 203, 211),
    (64, 256, 256, 256), (65, 384, 392, 400), (129, 4100, 4104, 4112),
    (67, 200, 208, 208),       # vector loads and stores with a partial last K-block and an M tail
]
LHS_SHAPES += [(int(m), int(k), int(k), int(k)) for m, k in _golden.table("pages_quant_shapes.txt")]


@pytest.mark.parametrize("M,K,ldx,ldq", LHS_SHAPES, ids=lambda v: str(v))
def test_quantize_lhs_parity(M, K, ldx, ldq):
    xh = _rand_bf16((M, K), seed=M * 7 + K)
    x = bf16_view(M, K, ldx, xh)
    q = GuardedU8(M, K, ldq)
    Kb = _cdiv(K, 128)
    a_s = GuardedF32((Kb, M))
    bf.quantize_lhs(x, q.view, a_s.view)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_lhs(xh)
    q.check_untouched()
    a_s.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(a_s.host().view(np.uint32), os_.view(np.uint32))


# row strips (K % 16 == 0, aligned rows): partial last groups, K cut into chunks of K-blocks
# (5248: 41 blocks in chunks of 21 and 20; 12304: 97 in 4), ragged strips; the last two shapes
# are not eligible (ldq % 16 != 0, K % 16 != 0) and run the tile kernel under every setting
STRIP_SHAPES = [
    (130, 144, 144, 144), (257, 4112, 4112, 4112), (300, 5248, 5256, 5264), (33, 12304, 12304, 12304),
    (2, 640, 640, 640), (1000, 1280, 1288, 1296), (4096, 4096, 4096, 4096),
    (77, 1280, 1280, 1288), (50, 1160, 1160, 1168),
]


@pytest.mark.parametrize("M,K,ldx,ldq", STRIP_SHAPES, ids=lambda v: str(v))
def test_quantize_lhs_every_strip_size(M, K, ldx, ldq, monkeypatch):
    """Every strip size and the tile kernel (BSFP8_QUANT_LHS_STRIP = 0) give the oracle's codes and
    scales bit for bit, with nothing written outside the tensors."""
    xh = _rand_bf16((M, K), seed=M * 11 + K)
    oq, os_ = oracle.quantize_lhs(xh)
    x = bf16_view(M, K, ldx, xh)
    for setting in ("", "0", "1", "2", "4", "8", "16"):
        monkeypatch.setenv("BSFP8_QUANT_LHS_STRIP", setting)
        q = GuardedU8(M, K, ldq)
        a_s = GuardedF32((_cdiv(K, 128), M))
        bf.quantize_lhs(x, q.view, a_s.view)
        torch.cuda.synchronize()
        q.check_untouched()
        a_s.check_untouched()
        assert np.array_equal(q.host(), oq), setting
        assert np.array_equal(a_s.host().view(np.uint32), os_.view(np.uint32)), setting


def test_quantize_lhs_edge_values():
    """Zero and negative-zero groups (eps path), +-448 boundaries, subnormal-range products,
    huge and tiny magnitudes."""
    M, K = 8, 512
    g = np.random.Generator(np.random.PCG64(99))
    x = g.standard_normal((M, K))
    x[0, :128] = 0.0
    x[1, :] = -0.0
    x[2, :128] = g.standard_normal(128) * 1e-30
    x[3, :] = g.standard_normal(K) * 3e38 / 5
    x[4, 128:256] = 2.0 ** -126 * g.integers(-3, 4, 128)
    x[5, :128] = np.where(np.arange(128) == 3, 448.0, 2.0 ** -16)   # amax 448, tie products
    x[6, :] = 1.0
    x[6, 7] = -1.0
    x[7, 256:384] = np.where(g.random(128) < 0.5, 1e-12, -1e-12)
    xh = inputs.bf16_bits_from_f64(x)
    xh[1, :] = 0x8000  # exact -0.0
    q, s = bf.quantize_lhs(to_dev(xh))
    oq, os_ = oracle.quantize_lhs(xh)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_quantize_lhs_workloads_full_size(idx):
    d = inputs.make_workload(idx)
    for name in [k for k in d if k in ("A", "X", "dY")]:
        xh = d[name]
        q, s = bf.quantize_lhs(to_dev(xh))
        oq, os_ = oracle.quantize_lhs(xh)
        assert np.array_equal(q.cpu().numpy(), oq), name
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), name


# ------------------------------------------------------------------ quantize_rhs

RHS_SHAPES = [
    (128, 64, 64, 128), (130, 70, 72, 144), (300, 129, 136, 304), (1, 5, 5, 1),
    (256, 384, 390, 260), (4096, 1024, 1024, 4096), (2048, 8192, 8192, 2048),
    # more workgroups than one round of residents (65 x 33 > 8 per CU): K-block-fastest order,
    # with K and N tails and padded strides
    (8200, 2056, 2064, 8208),
    (208, 136, 136, 208),      # vector loads and stores, K and N tails
]


@pytest.mark.parametrize("K,N,ldx,ldqT", RHS_SHAPES, ids=lambda v: str(v))
def test_quantize_rhs_parity(K, N, ldx, ldqT):
    xh = _rand_bf16((K, N), seed=K * 3 + N)
    x = bf16_view(K, N, ldx, xh)
    qT = GuardedU8(N, K, ldqT)
    s = GuardedF32((_cdiv(K, 128), N))
    bf.quantize_rhs(x, qT.view, s.view)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_rhs(xh)
    qT.check_untouched()
    s.check_untouched()
    assert np.array_equal(qT.host(), oq)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))


def test_quantize_rhs_training_step_full_size():
    d = inputs.make_workload(3)
    for name in ("X", "dY"):
        xh = d[name]
        qT, s = bf.quantize_rhs(to_dev(xh))
        oq, os_ = oracle.quantize_rhs(xh)
        assert np.array_equal(qT.cpu().numpy(), oq), name
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), name


# ------------------------------------------------------------------ quantize_lhs_and_rhs

DUAL_SHAPES = [
    (128, 128, 128, 128, 128), (130, 1280, 1288, 1296, 144), (1, 1, 1, 1, 1),
    (257, 300, 304, 312, 272), (300, 129, 136, 144, 304), (129, 257, 264, 264, 129),
    (5, 200, 203, 211, 5), (2048, 2048, 2048, 2048, 2048), (384, 640, 640, 640, 390),
    (272, 264, 264, 272, 272),  # vector loads and both vector stores, R and C tails
]


@pytest.mark.parametrize("R,C,ldx,ldq,ldqT", DUAL_SHAPES, ids=lambda v: str(v))
def test_quantize_lhs_and_rhs_parity(R, C, ldx, ldq, ldqT):
    """One pass writes exactly the oracle's 1x128 row-wise and 128x1 transposed outputs; nothing
    outside them (sentinel rows/padding, NaN guard bands around both scale tensors)."""
    xh = _rand_bf16((R, C), seed=R * 7 + C)
    x = bf16_view(R, C, ldx, xh)
    q = GuardedU8(R, C, ldq)
    a_s = GuardedF32((_cdiv(C, 128), R))
    qT = GuardedU8(C, R, ldqT)
    s = GuardedF32((_cdiv(R, 128), C))
    bf.quantize_lhs_and_rhs(x, q.view, a_s.view, qT.view, s.view)
    torch.cuda.synchronize()
    oq, oas = oracle.quantize_lhs(xh)
    oqT, os_ = oracle.quantize_rhs(xh)
    for g in (q, a_s, qT, s):
        g.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(a_s.host().view(np.uint32), oas.view(np.uint32))
    assert np.array_equal(qT.host(), oqT)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))


def test_quantize_lhs_and_rhs_training_step_full_size():
    """X and dY of the training step [8192, 4096]: oracle parity, and equal bytes to the two
    single-purpose kernels."""
    d = inputs.make_workload(3)
    for name in ("X", "dY"):
        xh = d[name]
        x = to_dev(xh)
        q, a_s, qT, s = bf.quantize_lhs_and_rhs(x)
        oq, oas = oracle.quantize_lhs(xh)
        assert np.array_equal(q.cpu().numpy(), oq), name
        assert np.array_equal(a_s.cpu().numpy().view(np.uint32), oas.view(np.uint32)), name
        oqT, os_ = oracle.quantize_rhs(xh)
        assert np.array_equal(qT.cpu().numpy(), oqT), name
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), name
        q1, s1 = bf.quantize_lhs(x)
        q2, s2 = bf.quantize_rhs(x)
        assert torch.equal(q1, q) and torch.equal(s1.view(torch.int32), a_s.view(torch.int32)), name
        assert torch.equal(q2, qT) and torch.equal(s2.view(torch.int32), s.view(torch.int32)), name


def test_quantize_lhs_and_rhs_outliers_and_zero_groups():
    """Outlier columns and all-zero 1x128 groups (the eps clamp) through the fused kernel."""
    d = inputs.make_workload(4, scale_down=8, zero_groups=True)
    xh = d["A"]
    q, a_s, qT, s = bf.quantize_lhs_and_rhs(to_dev(xh))
    oq, oas = oracle.quantize_lhs(xh)
    oqT, os_ = oracle.quantize_rhs(xh)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), oas.view(np.uint32))
    assert np.array_equal(qT.cpu().numpy(), oqT)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


# ------------------------------------------------------------------ quantize_weight_128x128

W_SHAPES = [
    (512, 128, 128, 128, 512), (5120, 1280, 1280, 1280, 5120), (130, 300, 304, 312, 144),
    (5, 1, 8, 16, 16), (256, 257, 264, 272, 256), (129, 129, 130, 131, 133),
    (144, 264, 264, 272, 144),  # vector loads and stores (qT too), N and K tails
]


@pytest.mark.parametrize("N,K,ldw,ldq,ldqT", W_SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("want_qT", [True, False])
def test_quantize_weight_parity(N, K, ldw, ldq, ldqT, want_qT):
    wh = _rand_bf16((N, K), seed=N * 5 + K)
    w = bf16_view(N, K, ldw, wh)
    q = GuardedU8(N, K, ldq)
    qT = GuardedU8(K, N, ldqT) if want_qT else None
    s = GuardedF32((_cdiv(N, 128), _cdiv(K, 128)))
    bf.quantize_weight_128x128(w, q.view, qT.view if qT else None, s.view, want_qT=want_qT)
    torch.cuda.synchronize()
    oq, oqT, os_ = oracle.quantize_weight_128x128(wh)
    q.check_untouched()
    s.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))
    if qT:
        qT.check_untouched()
        assert np.array_equal(qT.host(), oqT)


@pytest.mark.parametrize("idx", [2, 4])
def test_quantize_weight_workloads_full_size(idx):
    wh = inputs.make_workload(idx)["W"]
    q, qT, s = bf.quantize_weight_128x128(to_dev(wh))
    oq, oqT, os_ = oracle.quantize_weight_128x128(wh)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(qT.cpu().numpy(), oqT)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
