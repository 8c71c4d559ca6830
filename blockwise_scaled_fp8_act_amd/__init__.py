"""Blockwise-scaled FP8 linear-layer kernels for MI355X (gfx950).

Group quantizers (1x128, 128x1, 128x128, and 1x128 + 128x1 of one tensor in a single pass) from
bf16 to float8_e4m3fn (or float8_e4m3fnuz, ``fmt="e4m3fnuz"``) with fp32 scales, and the
1x128 x 128x128 / 1x128 x 128x1 scaled FP8 GEMMs with bf16 output, as hand-written HIP kernels
behind the C ABI of include/blockwise_fp8.h. This package is the thin Python binding over that
library (``binding``), the blockwise-FP8 linear layer composed from those kernels for training
(``linear``), its in-tree build (``build``) and the seeded input generators (``inputs``).
"""
from .binding import (  # noqa: F401
    Bsfp8Error,
    encode_e4m3_f32,
    encode_e4m3fnuz_f32,
    fp8_format,
    gemm_1x128_128x1,
    gemm_1x128_128x1_grouped,
    gemm_1x128_128x128,
    gemm_1x128_128x128_grouped,
    gemm_1x128_128x128_noalloc,
    quantize_lhs,
    quantize_lhs_and_rhs,
    quantize_lhs_and_weight,
    quantize_rhs,
    quantize_rhs_grouped,
    quantize_weight_128x128,
)
from .linear import BlockwiseFp8Linear, blockwise_fp8_linear  # noqa: F401
