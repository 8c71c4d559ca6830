"""Seeded synthetic inputs for the blockwise FP8 linear-layer workloads.

This module only draws random tensors and rounds them to bf16; it holds none of the quantize or
GEMM arithmetic, so both the HIP path's tests/benchmark and the CPU oracle's tests can use it.

Recipe (the same for every workload):
  * ``numpy.random.Generator(PCG64(seed))``, seed 0 unless stated;
  * draws are fp64, rounded to fp32 and then to bf16 with round-to-nearest-even;
  * draw order inside a workload: activation (A or X), weight W, output gradient dY, then any
    selection draws (outlier columns, zeroed groups);
  * activations are [tokens, features]; weights are [N_out, K_in] (nn.Linear layout).

Workloads mirror the pages' shapes (the quantization-correctness, SQNR and performance tables of
"Enable blockwise FP8 dense training kernels on ROCm"): small and tail-masking GEMMs, the 4096^3
forward GEMM, one linear-layer training step, and an outlier-heavy activation case.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_f64(x) -> np.ndarray:
    """fp64 -> fp32 (IEEE round to nearest) -> bf16 bit pattern (round to nearest, ties to even)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return bf16_bits_from_f64(g.standard_normal(shape) * std)


def _apply_outliers(g: np.random.Generator, a: np.ndarray, n_channels: int, zero_frac: float,
                    zero_whole_groups: bool) -> np.ndarray:
    """Multiply n_channels random K-channels by 100, then set a zero_frac share to exactly zero:
    single elements drawn at random over the tensor, or (zero_whole_groups) whole 1x128 groups,
    whose all-zero amax takes the eps clamp."""
    M, K = a.shape
    cols = g.choice(K, size=n_channels, replace=False)
    a[:, cols] *= 100.0
    if not zero_whole_groups:
        n_zero = int(round(zero_frac * M * K))
        flat = g.choice(M * K, size=n_zero, replace=False)
        a.reshape(-1)[flat] = 0.0
        return a
    kb = (K + BLOCK - 1) // BLOCK
    n_groups = M * kb
    n_zero = int(round(zero_frac * n_groups))
    groups = g.choice(n_groups, size=n_zero, replace=False)
    for gid in groups:
        m, b = divmod(int(gid), kb)
        a[m, b * BLOCK:(b + 1) * BLOCK] = 0.0
    return a


WORKLOADS = {
    0: "fwd_small: A[2,128]~N(0,1), W drawn [128,512]~N(0,0.02^2) then used as [512,128]",
    1: "fwd_tail: A[130,1280]~N(0,1), W[5120,1280]~N(0,0.02^2)",
    2: "fwd_4096: A[4096,4096]~N(0,1), W[4096,4096]~N(0,0.02^2)",
    3: "train_step: X[8192,4096]~N(0,1), W[4096,4096]~N(0,0.02^2), dY[8192,4096]~N(0,0.01^2)",
    4: "fwd_outlier: A[16384,5120]~N(0,1) with 26 columns x100 and 1% of elements exactly zero, "
       "W[5120,5120]~t(4)*0.02 (zero_groups=True: 1% of whole 1x128 groups zero instead, the eps "
       "clamp case)",
}


def make_workload(idx: int, seed: int = 0, scale_down: int = 1, zero_groups: bool = False) -> dict:
    """Return the named bf16 tensors (uint16 bit patterns) of workload ``idx``.

    ``scale_down`` > 1 divides the token dimension (and, for the outlier case, nothing else) so
    CPU-only tests can use the same recipe at a smaller size; the full size is scale_down = 1.
    ``zero_groups`` (outlier case only) zeroes 1% of whole 1x128 groups instead of 1% of the
    elements, so the eps clamp of an all-zero group is exercised.
    """
    g = rng(seed)
    if idx == 0:
        a = normal_bf16(g, (2, 128))
        w_kn = normal_bf16(g, (128, 512), 0.02)
        return {"A": a, "W": np.ascontiguousarray(w_kn.T)}
    if idx == 1:
        return {"A": normal_bf16(g, (130, 1280)), "W": normal_bf16(g, (5120, 1280), 0.02)}
    if idx == 2:
        return {"A": normal_bf16(g, (4096, 4096)), "W": normal_bf16(g, (4096, 4096), 0.02)}
    if idx == 3:
        T = 8192 // scale_down
        x = normal_bf16(g, (T, 4096))
        w = normal_bf16(g, (4096, 4096), 0.02)
        dy = normal_bf16(g, (T, 4096), 0.01)
        return {"X": x, "W": w, "dY": dy}
    if idx == 4:
        M, K, N = 16384 // scale_down, 5120, 5120
        a = g.standard_normal((M, K))
        w = g.standard_t(4.0, size=(N, K)) * 0.02
        a = _apply_outliers(g, a, n_channels=int(round(0.005 * K)), zero_frac=0.01,
                            zero_whole_groups=zero_groups)
        return {"A": bf16_bits_from_f64(a), "W": bf16_bits_from_f64(w)}
    raise ValueError(f"unknown workload {idx}")
