"""Blockwise-FP8 linear layer for training, composed from the C-ABI kernels.

"Enable blockwise FP8 dense training kernels on ROCm" names the parts but not their wiring: its
quantization-correctness table lists three quantizers (act_quant_lhs, act_quant_rhs,
weight_quant_rhs, block_size 128), its description mentions the blockwise linear module
(Float8BlockwiseLinear) and the dense training kernels, and "Mask a_s/b_s scale loads in blockwise
FP8 training GEMM kernels" names the two GEMMs (1x128_128x128, 1x128_128x1). Which quantizer feeds
which GEMM of a training step is this module's reading -- the one the groupings force, since the
1x128 and 128x128 groups run along the contracted dimension of the forward and dgrad products and
the 128x1 groups along the tokens the weight gradient contracts over:

    forward   Y  = X W^T      A = quantize_lhs(X)        (1x128 along in_features)
                              B = quantize_weight(W)     (128x128), gemm_1x128_128x128
    dgrad     dX = dY W       A = quantize_lhs(dY)       (1x128 along out_features)
                              B = quantize_weight(W)^T   (the transposed codes qT, same scales read
                                                          transposed), gemm_1x128_128x128
    wgrad     dW = dY^T X     A = quantize_rhs(dY)       (128x1 along tokens, transposed)
                              B = quantize_rhs(X)        (128x1 along tokens, transposed),
                                                          gemm_1x128_128x1

X and dY each feed two GEMMs, so each is quantized once by quantize_lhs_and_rhs (both groupings in
one pass). The FP8 element format is float8_e4m3fn by default; ``fmt="e4m3fnuz"`` (or
torch.float8_e4m3fnuz) runs every quantizer and GEMM in float8_e4m3fnuz with FP8_MAX 240, the
dtype choice the same page adds for MI300X. Every step runs in the library's kernels; this module only allocates outputs, orders the
calls and keeps the forward's quantized operands for the backward (torch.autograd plumbing). All
tensors are bf16 on the GPU; outputs are bf16.
"""
from __future__ import annotations

import torch

from . import binding as _b


def _codes(rows: int, cols: int, device) -> torch.Tensor:
    """A [rows, cols] fp8-code buffer whose row stride is rounded up to 16 bytes, the alignment the
    GEMMs require of their operands (any token or feature count then works)."""
    ld = (cols + 15) // 16 * 16
    return torch.empty((rows, ld), dtype=torch.uint8, device=device)[:, :cols]


def _quantize_act(t: torch.Tensor, fmt: str):
    R, C = t.shape
    return _b.quantize_lhs_and_rhs(t, q=_codes(R, C, t.device), qT=_codes(C, R, t.device), fmt=fmt)


class _BlockwiseFp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, fmt: str) -> torch.Tensor:
        if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
            raise TypeError("blockwise FP8 linear expects bf16 activations and weights")
        if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
            raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w {tuple(w.shape)}")
        x = x.contiguous()
        w = w.contiguous()
        qx, sx, qxT, sxT = _quantize_act(x, fmt)
        need_dgrad = ctx.needs_input_grad[0]
        d_out, d_in = w.shape
        qw, qwT, sw = _b.quantize_weight_128x128(
            w, q=_codes(d_out, d_in, w.device), qT=_codes(d_in, d_out, w.device) if need_dgrad else None,
            want_qT=need_dgrad, fmt=fmt)
        y = _b.gemm_1x128_128x128(qx, sx, qw, sw, fmt=fmt)
        ctx.save_for_backward(qxT, sxT, qwT if need_dgrad else None, sw)
        ctx.shapes = (x.shape[0], x.shape[1], w.shape[0])
        ctx.fmt = fmt
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        qxT, sxT, qwT, sw = ctx.saved_tensors
        T, d_in, d_out = ctx.shapes
        fmt = ctx.fmt
        dy = dy.to(torch.bfloat16).contiguous()
        qdy, sdy, qdyT, sdyT = _quantize_act(dy, fmt)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            # B = W^T codes [d_in, d_out]; its (K-block over d_out, N-block over d_in) scale is the
            # weight scale s[kb][nb] of the [d_out/128, d_in/128] tensor: strides (1, d_in blocks)
            dx = _b.gemm_1x128_128x128(qdy, sdy, qwT, sw, 1, sw.shape[1], fmt=fmt)
        if ctx.needs_input_grad[1]:
            dw = _b.gemm_1x128_128x1(qdyT, sdyT, qxT, sxT, fmt=fmt)
        return dx, dw, None


def blockwise_fp8_linear(x: torch.Tensor, w: torch.Tensor, fmt="e4m3fn") -> torch.Tensor:
    """Y = X W^T (no bias) with the blockwise-FP8 forward and backward; x [T, in], w [out, in].
    ``fmt``: FP8 element format ("e4m3fn", "e4m3fnuz" or the torch float8 dtype)."""
    return _BlockwiseFp8LinearFn.apply(x, w, _b.fp8_format(fmt))


class BlockwiseFp8Linear(torch.nn.Module):
    """nn.Linear replacement (bf16 parameters) whose forward and backward GEMMs run in blockwise
    FP8. A bias, if any, is added in bf16 after the FP8 GEMM."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False, device=None,
                 fmt="e4m3fn"):
        super().__init__()
        self.in_features, self.out_features = in_features, out_features
        self.fmt = _b.fp8_format(fmt)
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device))
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16, device=device))
                     if bias else None)
        torch.nn.init.normal_(self.weight, std=0.02)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        y = blockwise_fp8_linear(x.reshape(-1, self.in_features), self.weight, self.fmt)
        if self.bias is not None:
            y = y + self.bias
        return y.reshape(*lead, self.out_features)
