"""The Python binding rejects malformed tensors before calling the library: wrong dtype, rank,
shape or row layout raise TypeError / ValueError, and tensors that are not on the current GPU raise
ValueError. Runs without a GPU (every case fails before the library is touched)."""
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf

BF = torch.bfloat16
U8 = torch.uint8
F32 = torch.float32


def _x(M=4, K=256, dtype=BF):
    return torch.zeros((M, K), dtype=dtype)


@pytest.mark.parametrize("fn", [bf.quantize_lhs, bf.quantize_rhs, bf.quantize_lhs_and_rhs,
                                bf.quantize_weight_128x128])
def test_quantizers_reject_float32_input(fn):
    with pytest.raises(TypeError, match="dtype"):
        fn(_x(dtype=F32))


@pytest.mark.parametrize("fn", [bf.quantize_lhs, bf.quantize_rhs, bf.quantize_weight_128x128])
def test_quantizers_reject_1d_input(fn):
    with pytest.raises(ValueError, match="2-D"):
        fn(torch.zeros(256, dtype=BF))


def test_quantizers_reject_column_major_input():
    x = torch.zeros((256, 4), dtype=BF).t()          # [4, 256] with stride (1, 4)
    with pytest.raises(ValueError, match="contiguous rows"):
        bf.quantize_lhs(x)


def test_quantize_lhs_output_shape_and_dtype():
    x = _x(4, 256)
    with pytest.raises(ValueError, match="q has shape"):
        bf.quantize_lhs(x, q=torch.zeros((4, 128), dtype=U8))
    with pytest.raises(TypeError, match="q has dtype"):
        bf.quantize_lhs(x, q=torch.zeros((4, 256), dtype=torch.int8))
    with pytest.raises(ValueError, match="a_s has shape"):
        bf.quantize_lhs(x, a_s=torch.zeros((4, 2), dtype=F32))     # (M, Kb): transposed
    with pytest.raises(ValueError, match="must be contiguous"):
        bf.quantize_lhs(x, a_s=torch.zeros((4, 2), dtype=F32).t())


def test_format_must_match_code_dtype():
    x = _x(4, 256)
    with pytest.raises(TypeError, match="q has dtype"):
        bf.quantize_lhs(x, q=torch.zeros((4, 256), dtype=torch.float8_e4m3fnuz))
    with pytest.raises(ValueError, match="unsupported FP8 format"):
        bf.quantize_lhs(x, fmt="e5m2")


def test_quantize_rhs_and_weight_output_shapes():
    x = _x(256, 8)
    with pytest.raises(ValueError, match="qT has shape"):
        bf.quantize_rhs(x, qT=torch.zeros((256, 8), dtype=U8))
    with pytest.raises(ValueError, match="s has shape"):
        bf.quantize_rhs(x, s=torch.zeros((8, 2), dtype=F32))
    w = _x(256, 384)
    with pytest.raises(ValueError, match="qT has shape"):
        bf.quantize_weight_128x128(w, qT=torch.zeros((256, 384), dtype=U8))
    with pytest.raises(ValueError, match="s has shape"):
        bf.quantize_weight_128x128(w, s=torch.zeros((3, 2), dtype=F32))


def test_cpu_tensors_are_rejected():
    """Well-formed tensors in host memory: the library reads device pointers only."""
    with pytest.raises(ValueError, match="GPU tensor"):
        bf.quantize_lhs(_x(4, 256))
    with pytest.raises(ValueError, match="GPU tensor"):
        bf.quantize_lhs_and_weight(_x(4, 256), _x(128, 256))


def _gemm_args(M=4, N=256, K=256):
    a = torch.zeros((M, K), dtype=U8)
    b = torch.zeros((N, K), dtype=U8)
    a_s = torch.ones(((K + 127) // 128, M), dtype=F32)
    b_s = torch.ones(((N + 127) // 128, (K + 127) // 128), dtype=F32)
    return a, a_s, b, b_s


def test_gemm_checks():
    a, a_s, b, b_s = _gemm_args()
    with pytest.raises(TypeError, match="a has dtype"):
        bf.gemm_1x128_128x128(a.to(torch.int8), a_s, b, b_s)
    with pytest.raises(ValueError, match="a_s has shape"):
        bf.gemm_1x128_128x128(a, a_s.t().contiguous(), b, b_s)
    with pytest.raises(ValueError, match="K = 300"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s, K=300)
    with pytest.raises(ValueError, match="b_s holds"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s, 3, 1)                # strides read past b_s
    with pytest.raises(ValueError, match=">= 0"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s, -1, 1)
    with pytest.raises(ValueError, match="c has shape"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s, c=torch.zeros((4, 128), dtype=BF))
    with pytest.raises(TypeError, match="c has dtype"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s, c=torch.zeros((4, 256), dtype=F32))
    with pytest.raises(ValueError, match="GPU tensor"):
        bf.gemm_1x128_128x128(a, a_s, b, b_s)
    with pytest.raises(ValueError, match="GPU tensor"):
        bf.gemm_1x128_128x128_noalloc(a, a_s, b, b_s, torch.zeros((4, 256), dtype=BF))


def test_gemm_128x1_checks():
    a, a_s, b, _ = _gemm_args()
    with pytest.raises(ValueError, match="b_s has shape"):
        bf.gemm_1x128_128x1(a, a_s, b, torch.ones((2, 2), dtype=F32))
    with pytest.raises(ValueError, match="GPU tensor"):
        bf.gemm_1x128_128x1(a, a_s, b, torch.ones((2, 256), dtype=F32))


def test_grouped_checks():
    a, a_s, b, b_s = _gemm_args(M=8, N=256, K=256)
    off32 = torch.tensor([0, 4, 8], dtype=torch.int32)
    with pytest.raises(TypeError, match="offsets"):
        bf.gemm_1x128_128x128_grouped(a, a_s, b, b_s, off32, 2, 0, 0, 2, 1, N=128)
    with pytest.raises(ValueError, match="E \\+ 1"):
        bf.gemm_1x128_128x128_grouped(a, a_s, b, b_s, torch.tensor([0, 8]), 2, 0, 0, 2, 1, N=128)
    bT = torch.zeros((256, 256), dtype=U8)
    sT = torch.ones((2, 256), dtype=F32)
    with pytest.raises(ValueError, match="expected c"):
        bf.gemm_1x128_128x1_grouped(bT, sT, bT, sT, torch.tensor([0, 128, 256]), 2,
                                    c=torch.zeros((256, 256), dtype=BF))


def test_encode_checks():
    with pytest.raises(TypeError, match="float32"):
        bf.encode_e4m3_f32(torch.zeros(16, dtype=torch.float64))
    with pytest.raises(ValueError, match="uint8"):
        bf.encode_e4m3_f32(torch.zeros(16, dtype=F32), q=torch.zeros(8, dtype=U8))
