"""Pins for the oracle's float8_e4m3fnuz path (CPU only): the FP8_MAX = 240 parameterization of
"Enable blockwise FP8 dense training kernels on ROCm" (description: limits follow
torch.finfo(dtype), both e4m3fn and e4m3fnuz accepted; MI300X test log: FP8 max = 240).

The codec is pinned against torch's CPU float8_e4m3fnuz cast (exhaustively over every binary32
bit pattern, after clamping to +-240) and its decode table, and against brute-force nearest-value
search; the quantizers against hand-worked groups (tests/golden/hand_groups_fnuz.txt), invariants
and transposition identities; the GEMM against a closed form and a brute-force sum whose element
values come from torch's decode of the format.
"""
import numpy as np
import pytest
import torch

import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests import _golden

FMT = "e4m3fnuz"
ALL_CODES = np.arange(256, dtype=np.uint8)
FINITE_CODES = ALL_CODES[ALL_CODES != 0x80]
EPS = np.float32(1e-12)
F240 = np.float32(240.0)


def _torch_decode(codes):
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return torch.from_numpy(c.copy()).view(torch.float8_e4m3fnuz).to(torch.float64).numpy()


def _torch_encode(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(
        torch.float8_e4m3fnuz).view(torch.uint8).numpy()


# ------------------------------------------------------------------ codec

def test_decode_matches_torch_for_every_code():
    ours = oracle.fp8_decode(ALL_CODES, FMT)
    ref = _torch_decode(ALL_CODES)
    assert np.isnan(ours[0x80]) and np.isnan(ref[0x80])
    assert np.count_nonzero(np.isnan(ours)) == 1
    assert np.array_equal(ours[FINITE_CODES], ref[FINITE_CODES])


def test_format_constants():
    d = lambda c: oracle.fp8_decode(np.array([c]), FMT)[0]  # noqa: E731
    assert d(0x7F) == 240.0 and d(0xFF) == -240.0          # largest finite
    assert d(0x08) == 2.0 ** -7                             # smallest normal
    assert d(0x01) == 2.0 ** -10                            # smallest subnormal
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert oracle.FP8_MAX[FMT] == 240.0


def test_decode_relation_to_e4m3fn():
    """Same bit layout, exponent bias one higher: every code that is finite in both formats decodes
    to half its e4m3fn value (0x80 is -0 there and NaN here; 0x7F/0xFF NaN there, +-240 here)."""
    both = np.array([c for c in range(256) if c != 0x80 and (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.fp8_decode(both, FMT) * 2.0, oracle.e4m3_decode(both))


def test_roundtrip_every_finite_code():
    vals = oracle.fp8_decode(FINITE_CODES, FMT).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(vals, FMT), FINITE_CODES)


def test_encode_is_nearest_ties_to_even_bruteforce():
    g = np.random.Generator(np.random.PCG64(17))
    v = np.concatenate([
        g.uniform(-240, 240, 20000),
        g.standard_normal(20000) * np.exp2(g.integers(-15, 7, 20000)),
    ]).astype(np.float32)
    table_vals = oracle.fp8_decode(FINITE_CODES, FMT)
    pos = np.sort(table_vals[table_vals > 0])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, [np.float32(2.0 ** -11), np.float32(-2.0 ** -11)]])
    v = v.astype(np.float32)
    codes = oracle.fp8_encode(v, FMT)
    dist = np.abs(v.astype(np.float64)[:, None] - table_vals[None, :])
    best = dist.min(axis=1)
    got = np.abs(v.astype(np.float64) - oracle.fp8_decode(codes, FMT))
    assert np.array_equal(got, best)
    tie = (dist == best[:, None]).sum(axis=1) > 1
    # at a tie the chosen code has an even mantissa field (zero counts as even: 0x00)
    assert tie.sum() > 100
    assert np.all((codes[tie] & 1) == 0)
    assert not np.any(codes == 0x80), "the NaN pattern must never be produced"


def test_encode_saturates_and_has_no_negative_zero():
    v = np.array([240.0, 241.0, 247.9, 248.0, 500.0, 3e38, -1e30, -240.5,
                  -0.0, -1e-30, -2.0 ** -12], dtype=np.float32)
    assert list(oracle.fp8_encode(v, FMT)) == [0x7F] * 6 + [0xFF, 0xFF] + [0x00] * 3


@pytest.mark.parametrize("chunk", range(64))
def test_encode_exhaustive_vs_torch(chunk):
    """All 2^32 binary32 patterns (64 chunks of 2^26): the oracle's saturating encoder equals
    torch's RNE cast applied after clamping to +-240 (torch turns overflow into NaN instead).
    NaN inputs are outside the contract and skipped."""
    n = 1 << 26
    first = chunk * n
    ours = oracle.fp8_encode_bits(first, n, FMT)
    bits = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    ok = ~np.isnan(f)
    ref = _torch_encode(np.clip(f, -F240, F240))
    bad = np.nonzero((ours != ref) & ok)[0]
    assert bad.size == 0, f"first mismatch at bits {hex(first + int(bad[0]))}"


# ------------------------------------------------------------------ quantizers

@pytest.mark.parametrize("case", _golden.hand_groups("hand_groups_fnuz.txt"),
                         ids=lambda c: c["name"])
def test_hand_worked_group(case):
    row = np.full(128, case["fill"], dtype=np.float64)
    row[: len(case["x"])] = case["x"]
    bits = inputs.bf16_bits_from_f64(row)
    assert np.array_equal(inputs.bf16_bits_to_f32(bits).astype(np.float64), row)
    q, a_s = oracle.quantize_lhs(bits[None, :], fmt=FMT)
    assert int(a_s.view(np.uint32)[0, 0]) == case["s_bits"]
    n = len(case["q"])
    assert [int(c) for c in q[0, :n]] == case["q"]
    assert np.all(q[0, n:] == 0x00)
    # the same group seen by the 128x1 quantizer (a column) and inside a 128x128 block
    qT, s = oracle.quantize_rhs(bits[:, None].copy(), fmt=FMT)
    assert np.array_equal(qT[0], q[0]) and s.view(np.uint32)[0, 0] == case["s_bits"]


def _random_rows(M, K, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    mag = np.exp2(g.integers(-30, 30, size=(M, 1)).astype(np.float64))
    return inputs.bf16_bits_from_f64(g.standard_normal((M, K)) * mag)


def test_invariants_random_groups():
    x = _random_rows(257, 384, 3)
    x[5, :128] = 0                                        # an all-zero group
    q, a_s = oracle.quantize_lhs(x, fmt=FMT)
    assert not np.any(q == 0x80)
    dec = oracle.fp8_decode(q, FMT)
    assert np.all(np.abs(dec) <= 240.0)
    xf = inputs.bf16_bits_to_f32(x).reshape(257, 3, 128)
    amax = np.abs(xf).max(axis=2)
    amax_c = np.maximum(amax, EPS).astype(np.float32)
    # stored scale: one IEEE fp32 division amax_c / 240 (column-major [M, Kb] as (Kb, M))
    assert np.array_equal(a_s.T, (amax_c / F240).astype(np.float32))
    # every group with amax >= eps holds a +-240 code
    top = (np.abs(dec.reshape(257, 3, 128)) == 240.0).any(axis=2)
    assert np.array_equal(top, amax >= EPS)
    # dequantized values stay within half a code step (plus the fp32 product rounding) of x
    deq = dec.reshape(257, 3, 128) * a_s.T[:, :, None].astype(np.float64)
    err = np.abs(deq - xf)
    assert np.all(err <= np.abs(xf) * (2.0 ** -4 + 2.0 ** -20) + a_s.T[:, :, None] * 2.0 ** -11)


def test_rhs_is_transposed_lhs():
    x = _random_rows(300, 200, 4)          # [K=300 tokens, N=200], ragged in both
    qT, s = oracle.quantize_rhs(x, fmt=FMT)
    q2, a_s2 = oracle.quantize_lhs(np.ascontiguousarray(x.T), fmt=FMT)
    assert np.array_equal(qT, q2)
    assert np.array_equal(s, a_s2)


def test_weight_transpose_identity():
    g = np.random.Generator(np.random.PCG64(5))
    w = inputs.bf16_bits_from_f64(g.standard_t(4, size=(300, 260)) * 0.02)
    q, qT, s = oracle.quantize_weight_128x128(w, fmt=FMT)
    q2, qT2, s2 = oracle.quantize_weight_128x128(np.ascontiguousarray(w.T), fmt=FMT)
    assert np.array_equal(qT, q.T) and np.array_equal(q2, qT) and np.array_equal(qT2, q)
    assert np.array_equal(s2, s.T)
    assert not np.any(q == 0x80)


# ------------------------------------------------------------------ GEMM

def test_gemm_closed_form():
    """All codes 0x40 (= 1.0 in e4m3fnuz), a_s = alpha, b_s = beta: C = alpha beta K."""
    M, N, K = 5, 131, 300
    a = np.full((M, K), 0x40, dtype=np.uint8)
    b = np.full((N, K), 0x40, dtype=np.uint8)
    Kb = oracle.cdiv(K, 128)
    a_s = np.full((Kb, M), 0.375, dtype=np.float32)
    b_s = np.full((2, Kb), 0.0625, dtype=np.float32)
    c = oracle.gemm_1x128_128x128(a, a_s, b, b_s, Kb, 1, fmt=FMT)
    assert np.all(c == 0.375 * 0.0625 * K)
    bcol = np.full((Kb, N), 0.0625, dtype=np.float32)
    assert np.all(oracle.gemm_1x128_128x1(a, a_s, b, bcol, fmt=FMT) == 0.375 * 0.0625 * K)


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (4, 130, 200), (9, 17, 385)])
def test_gemm_bruteforce_with_torch_decode(M, N, K):
    """Blockwise form == direct sum over k of (A[m,k] a_s[m,kb]) (B[n,k] b_s(kb,n)), the element
    values taken from torch's float8_e4m3fnuz decode."""
    g = np.random.Generator(np.random.PCG64(M * N + K))
    a = g.choice(FINITE_CODES, size=(M, K)).astype(np.uint8)
    b = g.choice(FINITE_CODES, size=(N, K)).astype(np.uint8)
    Kb = oracle.cdiv(K, 128)
    Nb = oracle.cdiv(N, 128)
    a_s = np.exp2(g.integers(-8, 8, size=(Kb, M))).astype(np.float32)
    b_s = np.exp2(g.integers(-8, 8, size=(Nb, Kb))).astype(np.float32)
    bcol = np.exp2(g.integers(-8, 8, size=(Kb, N))).astype(np.float32)
    av, bv = _torch_decode(a), _torch_decode(b)
    kb_of = np.arange(K) // 128
    sa = a_s.T[:, kb_of].astype(np.float64)                      # [M, K]
    sb = b_s[np.arange(N) // 128][:, kb_of].astype(np.float64)   # [N, K]
    ref = (av * sa) @ (bv * sb).T
    assert np.allclose(oracle.gemm_1x128_128x128(a, a_s, b, b_s, Kb, 1, fmt=FMT), ref,
                       rtol=1e-12, atol=0)
    sbc = bcol.T[:, kb_of].astype(np.float64)
    ref = (av * sa) @ (bv * sbc).T
    assert np.allclose(oracle.gemm_1x128_128x1(a, a_s, b, bcol, fmt=FMT), ref, rtol=1e-12, atol=0)


def test_gemm_fnuz_equals_fn_on_halved_codes():
    """Codes valid in both formats, fnuz value = e4m3fn value / 2: the fnuz GEMM equals the e4m3fn
    GEMM on the same codes with a_s and b_s each halved."""
    g = np.random.Generator(np.random.PCG64(9))
    both = np.array([c for c in range(256) if c != 0x80 and (c & 0x7F) != 0x7F], dtype=np.uint8)
    M, N, K = 6, 140, 260
    a = g.choice(both, size=(M, K)).astype(np.uint8)
    b = g.choice(both, size=(N, K)).astype(np.uint8)
    Kb = oracle.cdiv(K, 128)
    a_s = g.uniform(0.5, 2, size=(Kb, M)).astype(np.float32)
    b_s = g.uniform(0.5, 2, size=(2, Kb)).astype(np.float32)
    c_nuz = oracle.gemm_1x128_128x128(a, a_s, b, b_s, Kb, 1, fmt=FMT)
    c_fn = oracle.gemm_1x128_128x128(a, a_s / 2, b, b_s / 2, Kb, 1)
    assert np.array_equal(c_nuz, c_fn)
