"""GPU parity of quantize_lhs_and_weight, the forward step's two quantizations in one launch: the
1x128 row-wise groups of the activation and the 128x128 blocks of the weight ("Enable blockwise
FP8 dense training kernels on ROCm", quantization-correctness table: act_quant_lhs and
weight_quant_rhs). Codes and scales must equal the oracle's bit for bit, in guard-banded outputs,
on shapes with ragged edges in every direction, with and without the transposed weight copy, in
both element formats, and on strides that send the call to the two single-purpose kernels.
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests._gpu import GuardedF32, GuardedU8, bf16_view

pytestmark = pytest.mark.gpu


def _cdiv(a, b):
    return (a + b - 1) // b


def _rand_bf16(shape, seed, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape) * scale * np.exp2(g.integers(-12, 12, size=(shape[0], 1)))
    return inputs.bf16_bits_from_f64(x)


# M, K, ldx, N, Kw, ldw, want_qT: 16-byte rows (one persistent launch) unless noted
STEP_SHAPES = [
    (4096, 4096, 4096, 4096, 4096, 4096, False),   # the forward step's shapes
    (2, 128, 128, 512, 128, 128, False),           # small forward case
    (130, 1280, 1280, 5120, 1280, 1280, True),     # M tail, weight with qT
    (300, 200, 208, 130, 300, 304, True),          # ragged K, N and Kw (Kw % 8 != 0: two kernels)
    (300, 200, 208, 144, 296, 304, True),          # ragged K, N and Kw in one launch
    (2100, 4000, 4008, 2192, 4000, 4008, True),    # several tiles per workgroup, every edge ragged
    (5, 7, 8, 3, 9, 16, False),                    # sub-group sizes
    (129, 256, 263, 256, 129, 131, True),          # odd strides: the two single-purpose kernels
    # without the transposed copy (reads and writes in separate phases): ragged edges, several
    # tiles per workgroup, and two runs of tiles per workgroup
    (300, 200, 208, 144, 296, 304, False),
    (2100, 4000, 4008, 2192, 4000, 4008, False),
    (8192, 4096, 4096, 4096, 4096, 4096, False),
]


def _run(M, K, ldx, N, Kw, ldw, want_qT, fmt, seed):
    xh = _rand_bf16((M, K), seed)
    wh = _rand_bf16((N, Kw), seed + 1, 0.02)
    x = bf16_view(M, K, ldx, xh)
    w = bf16_view(N, Kw, ldw, wh)
    ld16 = lambda n: (n + 15) // 16 * 16  # noqa: E731
    qx = GuardedU8(M, K, ld16(K))
    sx = GuardedF32((_cdiv(K, 128), M))
    qw = GuardedU8(N, Kw, ld16(Kw))
    qwT = GuardedU8(Kw, N, ld16(N)) if want_qT else None
    sw = GuardedF32((_cdiv(N, 128), _cdiv(Kw, 128)))
    bf.quantize_lhs_and_weight(x, w, qx.view, sx.view, qw.view, qwT.view if qwT else None, sw.view,
                               want_qT=want_qT, fmt=fmt)
    torch.cuda.synchronize()
    oqx, osx = oracle.quantize_lhs(xh, fmt=fmt)
    oqw, oqwT, osw = oracle.quantize_weight_128x128(wh, fmt=fmt)
    for g in (qx, sx, qw, sw) + ((qwT,) if qwT else ()):
        g.check_untouched()
    assert np.array_equal(qx.host(), oqx), "activation codes"
    assert np.array_equal(sx.host().view(np.uint32), osx.view(np.uint32)), "activation scales"
    assert np.array_equal(qw.host(), oqw), "weight codes"
    assert np.array_equal(sw.host().view(np.uint32), osw.view(np.uint32)), "weight scales"
    if qwT:
        assert np.array_equal(qwT.host(), oqwT), "transposed weight codes"


@pytest.mark.parametrize("M,K,ldx,N,Kw,ldw,want_qT", STEP_SHAPES, ids=lambda v: str(v))
def test_quantize_lhs_and_weight_parity(M, K, ldx, N, Kw, ldw, want_qT):
    _run(M, K, ldx, N, Kw, ldw, want_qT, "e4m3fn", seed=M + 3 * K + N)


@pytest.mark.parametrize("shape", [STEP_SHAPES[2], STEP_SHAPES[3], STEP_SHAPES[4]], ids=lambda v: str(v))
def test_quantize_lhs_and_weight_fnuz_parity(shape):
    _run(*shape, "e4m3fnuz", seed=17)


def test_quantize_lhs_and_weight_one_side_empty():
    """An empty activation or weight: the other tensor is quantized exactly as on its own."""
    wh = _rand_bf16((256, 384), 3, 0.02)
    w = bf16_view(256, 384, 384, wh)
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    _, _, qw, _, sw = bf.quantize_lhs_and_weight(x, w)
    oqw, _, osw = oracle.quantize_weight_128x128(wh, want_qT=False)
    assert np.array_equal(qw.cpu().numpy(), oqw) and np.array_equal(sw.cpu().numpy(), osw)
    xh = _rand_bf16((200, 300), 4)
    x = bf16_view(200, 300, 304, xh)
    w = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    qx, sx, _, _, _ = bf.quantize_lhs_and_weight(x, w)
    oqx, osx = oracle.quantize_lhs(xh)
    assert np.array_equal(qx.cpu().numpy(), oqx) and np.array_equal(sx.cpu().numpy(), osx)
