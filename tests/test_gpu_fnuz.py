"""GPU parity of the float8_e4m3fnuz entry points (FP8_MAX 240) against the oracle's e4m3fnuz path.

"Enable blockwise FP8 dense training kernels on ROCm" parameterizes FP8_MAX by the float8 dtype
and runs its MI300X checks in float8_e4m3fnuz; these tests hold the *_fnuz quantizers to the
oracle bit for bit (codes and scales, guard-banded outputs) and the *_fnuz GEMMs to the GEMM
tolerance (elementwise 2e-2 (|C_o| + 1), relative Frobenius 4e-3) on the oracle's own fnuz codes.
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests._gpu import DEV, GuardedF32, GuardedU8, bf16_view, to_dev

pytestmark = pytest.mark.gpu

FMT = "e4m3fnuz"
VALID = np.array([c for c in range(256) if c != 0x80], dtype=np.uint8)


def _cdiv(a, b):
    return (a + b - 1) // b


def _rand_bf16(shape, seed, spread=True):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape)
    if spread:
        x *= np.exp2(g.integers(-20, 20, size=(shape[0], 1)))
    return inputs.bf16_bits_from_f64(x)


def _check(c_gpu, c_oracle, what):
    rep = oracle.gemm_tolerance_report(c_gpu, c_oracle)
    assert rep["ok"], f"{what}: {rep}"


# ------------------------------------------------------------------ element conversion

# 2^28 bit patterns per chunk; chunks 0-4 hold every non-negative value up to 240 (1 + 2^-21)
# (0x43700007), chunks 8-12 the negative ones; the others hold only larger magnitudes or NaNs
@pytest.mark.parametrize("chunk", [0, 1, 2, 3, 4, 8, 9, 10, 11, 12])
def test_encode_fnuz_exhaustive_vs_oracle(chunk):
    """Every binary32 pattern with |v| <= 240 (1 + 2^-21): the quantizers' device conversion (the
    e4m3fn conversion of 2v, negative zero dropped) == the oracle's e4m3fnuz encoder of v."""
    n = 1 << 28
    first = chunk * n
    idx = torch.arange(first, first + n, dtype=torch.int64, device=DEV)
    idx = torch.where(idx >= 2 ** 31, idx - 2 ** 32, idx).to(torch.int32)
    x = idx.view(torch.float32)
    q = bf.encode_e4m3fnuz_f32(x)
    got = q.cpu().numpy()
    del idx, x, q
    ref = oracle.fp8_encode_bits(first, n, FMT)
    bits = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32)
    in_range = (bits & 0x7FFFFFFF) <= 0x43700007          # |v| <= 240 (1 + 2^-21), no NaN
    bad = np.nonzero((got != ref) & in_range)[0]
    assert in_range.any()
    assert bad.size == 0, (f"{bad.size} mismatches; first at bits {hex(first + int(bad[0]))}: "
                           f"gpu {got[bad[0]]:#x} oracle {ref[bad[0]]:#x}")
    assert not np.any(got[in_range] == 0x80)


# ------------------------------------------------------------------ quantizers

LHS_SHAPES = [(2, 128, 128, 128), (130, 1280, 1280, 1280), (3, 127, 128, 127),
              (65, 384, 392, 400), (129, 4100, 4104, 4112),
              (300, 5248, 5256, 5264), (4096, 4096, 4096, 4096)]  # row strips: chunked K, one round


@pytest.mark.parametrize("M,K,ldx,ldq", LHS_SHAPES, ids=lambda v: str(v))
def test_quantize_lhs_fnuz_parity(M, K, ldx, ldq):
    xh = _rand_bf16((M, K), seed=M * 3 + K)
    x = bf16_view(M, K, ldx, xh)
    q = GuardedU8(M, K, ldq)
    a_s = GuardedF32((_cdiv(K, 128), M))
    bf.quantize_lhs(x, q.view, a_s.view, fmt=FMT)
    torch.cuda.synchronize()
    oq, oas = oracle.quantize_lhs(xh, fmt=FMT)
    q.check_untouched()
    a_s.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(a_s.host().view(np.uint32), oas.view(np.uint32))


@pytest.mark.parametrize("K,N,ldx,ldqT", [(128, 64, 64, 128), (300, 200, 208, 304),
                                          (1, 5, 8, 16), (8192, 256, 256, 8192)],
                         ids=lambda v: str(v))
def test_quantize_rhs_fnuz_parity(K, N, ldx, ldqT):
    xh = _rand_bf16((K, N), seed=K + 5 * N)
    x = bf16_view(K, N, ldx, xh)
    qT = GuardedU8(N, K, ldqT)
    s = GuardedF32((_cdiv(K, 128), N))
    bf.quantize_rhs(x, qT.view, s.view, fmt=FMT)
    torch.cuda.synchronize()
    oqT, os_ = oracle.quantize_rhs(xh, fmt=FMT)
    qT.check_untouched()
    s.check_untouched()
    assert np.array_equal(qT.host(), oqT)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("N,K,ldw,ldq,ldqT",
                         [(512, 128, 128, 128, 512), (130, 300, 304, 312, 144),
                          (129, 129, 130, 131, 133)], ids=lambda v: str(v))
def test_quantize_weight_fnuz_parity(N, K, ldw, ldq, ldqT):
    wh = _rand_bf16((N, K), seed=N * 11 + K)
    w = bf16_view(N, K, ldw, wh)
    q = GuardedU8(N, K, ldq)
    qT = GuardedU8(K, N, ldqT)
    s = GuardedF32((_cdiv(N, 128), _cdiv(K, 128)))
    bf.quantize_weight_128x128(w, q.view, qT.view, s.view, fmt=FMT)
    torch.cuda.synchronize()
    oq, oqT, os_ = oracle.quantize_weight_128x128(wh, fmt=FMT)
    for g in (q, qT, s):
        g.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(qT.host(), oqT)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("R,C,ldx,ldq,ldqT",
                         [(130, 1280, 1288, 1296, 144), (257, 300, 304, 312, 272),
                          (2048, 2048, 2048, 2048, 2048)], ids=lambda v: str(v))
def test_quantize_lhs_and_rhs_fnuz_parity(R, C, ldx, ldq, ldqT):
    xh = _rand_bf16((R, C), seed=R + C)
    x = bf16_view(R, C, ldx, xh)
    q = GuardedU8(R, C, ldq)
    a_s = GuardedF32((_cdiv(C, 128), R))
    qT = GuardedU8(C, R, ldqT)
    s = GuardedF32((_cdiv(R, 128), C))
    bf.quantize_lhs_and_rhs(x, q.view, a_s.view, qT.view, s.view, fmt=FMT)
    torch.cuda.synchronize()
    oq, oas = oracle.quantize_lhs(xh, fmt=FMT)
    oqT, os_ = oracle.quantize_rhs(xh, fmt=FMT)
    for g in (q, a_s, qT, s):
        g.check_untouched()
    assert np.array_equal(q.host(), oq)
    assert np.array_equal(a_s.host().view(np.uint32), oas.view(np.uint32))
    assert np.array_equal(qT.host(), oqT)
    assert np.array_equal(s.host().view(np.uint32), os_.view(np.uint32))


def test_quantize_fnuz_outliers_zero_groups_and_negative_tiny():
    """Outlier columns, all-zero groups (eps clamp), and groups of -0.0 and of tiny negatives that
    round to zero: fnuz has no negative zero, so no 0x80 may appear."""
    d = inputs.make_workload(4, scale_down=8, zero_groups=True)
    xh = d["A"].copy()
    xh[0, :128] = 0x8000                                  # -0.0
    xh[1, :128] = inputs.bf16_bits_from_f64(np.full(128, -1e-30))
    xh[1, 0] = inputs.bf16_bits_from_f64(np.array([1.0]))[0]
    q, a_s = bf.quantize_lhs(to_dev(xh), fmt=FMT)
    oq, oas = oracle.quantize_lhs(xh, fmt=FMT)
    qh = q.cpu().numpy()
    assert np.array_equal(qh, oq)
    assert np.array_equal(a_s.cpu().numpy().view(np.uint32), oas.view(np.uint32))
    assert not np.any(qh == 0x80)
    assert np.all(qh[0, :128] == 0) and np.all(qh[1, 1:128] == 0) and qh[1, 0] == 0x7F


# ------------------------------------------------------------------ GEMMs

def _run_guarded(fn, M, N, ldc):
    cbuf = torch.full((M + 2, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    fn(cbuf[1:M + 1, :N])
    torch.cuda.synchronize()
    got = cbuf.float().cpu().numpy()
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[M + 1])), "write outside rows"
    assert np.all(np.isnan(got[1:M + 1, N:])), "write into row padding"
    return got[1:M + 1, :N]


def _padded(h, ld):
    buf = torch.zeros((h.shape[0], ld), dtype=torch.uint8, device=DEV)
    buf[:, :h.shape[1]] = torch.from_numpy(h).to(DEV)
    return buf[:, :h.shape[1]]


def test_gemm_fnuz_decodes_every_code():
    """A column of every valid fnuz code against 1.0 (0x40) with unit scales: C is the code's value,
    exact in bf16 (4 significant bits) -- on both operand sides."""
    M, N, K = 255, 130, 128
    a = np.zeros((M, K), dtype=np.uint8)
    a[:, 0] = VALID
    b = np.zeros((N, K), dtype=np.uint8)
    b[:, 0] = 0x40
    one_a = torch.ones((1, M), dtype=torch.float32, device=DEV)
    one_b = torch.ones((2, 1), dtype=torch.float32, device=DEV)
    c = bf.gemm_1x128_128x128(to_dev(a), one_a, to_dev(b), one_b, fmt=FMT)
    want = oracle.fp8_decode(VALID, FMT)
    assert np.array_equal(c.float().cpu().numpy(), np.repeat(want[:, None], N, axis=1))
    # B side, per-column scales: rows of 1.0 against the column of every code
    M2 = 7
    ones = np.zeros((M2, K), dtype=np.uint8)
    ones[:, 0] = 0x40
    c2 = bf.gemm_1x128_128x1(to_dev(ones), torch.ones((1, M2), device=DEV), to_dev(a),
                             torch.ones((1, M), device=DEV), fmt=FMT)
    assert np.array_equal(c2.float().cpu().numpy(), np.repeat(want[None, :], M2, axis=0))


GEMM_SHAPES = [
    (2, 512, 128, 128, 512), (130, 512, 1280, 1280, 512), (3, 5, 300, 304, 5),
    (129, 130, 129, 144, 131), (257, 384, 520, 528, 384), (300, 260, 256, 256, 262),
]


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x128_fnuz(M, N, K, ld, ldc):
    g = np.random.Generator(np.random.PCG64(M + N + K))
    ah = inputs.bf16_bits_from_f64(g.standard_normal((M, K)))
    wh = inputs.bf16_bits_from_f64(g.standard_normal((N, K)) * 0.02)
    oqa, osa = oracle.quantize_lhs(ah, fmt=FMT)
    oqw, _, osw = oracle.quantize_weight_128x128(wh, want_qT=False, fmt=FMT)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x128(_padded(oqa, ld), to_dev(osa),
                                                       _padded(oqw, ld), to_dev(osw), c=c, fmt=FMT),
                       M, N, ldc)
    co = oracle.gemm_1x128_128x128(oqa, osa, oqw, osw, osw.shape[1], 1, fmt=FMT)
    _check(got, co, "gemm_1x128_128x128_fnuz")
    ref = oracle.matmul_bf16_f64(ah, wh)
    assert oracle.sqnr_db(ref, got) >= 28.0  # the oracle's fnuz path: 28.66-30.39 dB on these shapes


@pytest.mark.parametrize("M,N,K,ld,ldc", GEMM_SHAPES, ids=lambda v: str(v))
def test_gemm_128x1_fnuz(M, N, K, ld, ldc):
    g = np.random.Generator(np.random.PCG64(M * N + K))
    dyh = inputs.bf16_bits_from_f64(g.standard_normal((K, M)) * 0.01)   # [tokens, M]
    xh = inputs.bf16_bits_from_f64(g.standard_normal((K, N)))           # [tokens, N]
    oqa, osa = oracle.quantize_rhs(dyh, fmt=FMT)     # A = dY^T codes [M, K], scales (Kb, M)
    oqb, osb = oracle.quantize_rhs(xh, fmt=FMT)      # B = X^T codes [N, K], scales (Kb, N)
    got = _run_guarded(lambda c: bf.gemm_1x128_128x1(_padded(oqa, ld), to_dev(osa),
                                                     _padded(oqb, ld), to_dev(osb), c=c, fmt=FMT),
                       M, N, ldc)
    co = oracle.gemm_1x128_128x1(oqa, osa, oqb, osb, fmt=FMT)
    _check(got, co, "gemm_1x128_128x1_fnuz")


def test_gemm_fnuz_4096_sampled():
    """The 4096^3 forward in fnuz: device quantizers (bit-exact), then the fnuz GEMM on sampled
    rows."""
    d = inputs.make_workload(2)
    a_h, w_h = d["A"], d["W"]
    qa, sa = bf.quantize_lhs(to_dev(a_h), fmt=FMT)
    qw, _, sw = bf.quantize_weight_128x128(to_dev(w_h), want_qT=False, fmt=FMT)
    c = bf.gemm_1x128_128x128(qa, sa, qw, sw, fmt=FMT)
    torch.cuda.synchronize()
    oqa, osa = oracle.quantize_lhs(a_h, fmt=FMT)
    oqw, _, osw = oracle.quantize_weight_128x128(w_h, want_qT=False, fmt=FMT)
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(sa.cpu().numpy(), osa)
    assert np.array_equal(qw.cpu().numpy(), oqw) and np.array_equal(sw.cpu().numpy(), osw)
    g = np.random.Generator(np.random.PCG64(0))
    rows = np.array(sorted(set(g.choice(4096, 48, replace=False).tolist()) | {0, 4095}))
    co = oracle.gemm_1x128_128x128(oqa, osa, oqw, osw, osw.shape[1], 1, rows=rows, fmt=FMT)
    cg = c.float().cpu().numpy()[rows]
    _check(cg, co, "fnuz forward 4096")
    ref = oracle.matmul_bf16_f64(a_h, w_h, rows=rows)
    assert oracle.sqnr_db(ref, cg) >= 28.0


def test_linear_layer_fnuz():
    """Forward and both backward GEMMs of the linear layer with fmt="e4m3fnuz" against the oracle
    composition in the same format (x [300, 256], W [384, 256]: ragged token count)."""
    g = np.random.Generator(np.random.PCG64(21))
    xh = inputs.bf16_bits_from_f64(g.standard_normal((300, 256)))
    wh = inputs.bf16_bits_from_f64(g.standard_normal((384, 256)) * 0.02)
    dyh = inputs.bf16_bits_from_f64(g.standard_normal((300, 384)) * 0.01)
    x = to_dev(xh).view(torch.bfloat16).requires_grad_(True)
    w = to_dev(wh).view(torch.bfloat16).requires_grad_(True)
    y = bf.blockwise_fp8_linear(x, w, fmt=torch.float8_e4m3fnuz)
    y.backward(to_dev(dyh).view(torch.bfloat16))
    torch.cuda.synchronize()
    qx, sx = oracle.quantize_lhs(xh, fmt=FMT)
    qw, qwT, sw = oracle.quantize_weight_128x128(wh, fmt=FMT)
    qdy, sdy = oracle.quantize_lhs(dyh, fmt=FMT)
    qxT, sxT = oracle.quantize_rhs(xh, fmt=FMT)
    qdyT, sdyT = oracle.quantize_rhs(dyh, fmt=FMT)
    kbw = sw.shape[1]
    _check(y.detach().float().cpu().numpy(),
           oracle.gemm_1x128_128x128(qx, sx, qw, sw, kbw, 1, fmt=FMT), "forward")
    _check(x.grad.float().cpu().numpy(),
           oracle.gemm_1x128_128x128(qdy, sdy, qwT, sw, 1, kbw, fmt=FMT), "dgrad")
    _check(w.grad.float().cpu().numpy(),
           oracle.gemm_1x128_128x1(qdyT, sdyT, qxT, sxT, fmt=FMT), "wgrad")


@pytest.mark.parametrize("per_col", [False, True], ids=["128x128", "128x1"])
def test_gemm_fnuz_partial_last_block_ignores_nan_padding(per_col):
    """Ragged K (300) with the NaN pattern 0x80 in every byte at and past K of the operand rows;
    the operands are the oracle's fnuz quantization of Gaussian data."""
    M, N, K, ld = 200, 136, 300, 320
    g = np.random.Generator(np.random.PCG64(5))
    ah, sa = oracle.quantize_lhs(inputs.bf16_bits_from_f64(g.standard_normal((M, K))), fmt=FMT)
    if per_col:
        bh, sb = oracle.quantize_rhs(inputs.bf16_bits_from_f64(g.standard_normal((K, N))), fmt=FMT)
    else:
        bh, _, sb = oracle.quantize_weight_128x128(
            inputs.bf16_bits_from_f64(g.standard_normal((N, K)) * 0.02), want_qT=False, fmt=FMT)

    def nan_padded(h):
        buf = torch.full((h.shape[0] + 1, ld), 0x80, dtype=torch.uint8, device=DEV)
        buf[:h.shape[0], :K] = torch.from_numpy(h).to(DEV)
        return buf[:h.shape[0], :K]

    a, b = nan_padded(ah), nan_padded(bh)
    if per_col:
        c = bf.gemm_1x128_128x1(a, to_dev(sa), b, to_dev(sb), fmt=FMT)
        co = oracle.gemm_1x128_128x1(ah, sa, bh, sb, fmt=FMT)
    else:
        c = bf.gemm_1x128_128x128(a, to_dev(sa), b, to_dev(sb), fmt=FMT)
        co = oracle.gemm_1x128_128x128(ah, sa, bh, sb, sb.shape[1], 1, fmt=FMT)
    got = c.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    _check(got, co, "fnuz partial last K-block")
