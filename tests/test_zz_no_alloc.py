"""GPU check of gemm_1x128_128x128_noalloc, the allocation-free form of gemm_1x128_128x128: its
K-split partial tiles live in the library's static scratch instead of an allocated workspace.

Two calls in a row, the second smaller, each against gemm_1x128_128x128 on the same operands (the
same kernels and split plan: bit-equal) and against the oracle (max |C - C_o| <= 2e-2 (|C_o| + 1)
elementwise, ||C - C_o||_F <= 4e-3 ||C_o||_F). The second call reads a scratch that still holds the
first call's partials, which must not leak into its result.
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests._gpu import DEV, to_dev

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = inputs.rng(seed)
    a_h = inputs.normal_bf16(g, (M, K))
    w_h = inputs.normal_bf16(g, (N, K), 0.02)
    qa, sa = bf.quantize_lhs(to_dev(a_h))
    qw, _, sw = bf.quantize_weight_128x128(to_dev(w_h), want_qT=False)
    torch.cuda.synchronize()
    oqa, osa = oracle.quantize_lhs(a_h)
    oqw, _, osw = oracle.quantize_weight_128x128(w_h, want_qT=False)
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(sa.cpu().numpy(), osa)
    assert np.array_equal(qw.cpu().numpy(), oqw) and np.array_equal(sw.cpu().numpy(), osw)
    return qa, sa, qw, sw, oqa, osa, oqw, osw


def _guarded(M, N):
    buf = torch.full((M + 2, N + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    return buf, buf[1:M + 1, :N]


def _check_guard(buf, M, N):
    h = buf.float().cpu().numpy()
    assert np.all(np.isnan(h[0])) and np.all(np.isnan(h[M + 1])) and np.all(np.isnan(h[1:M + 1, N:]))


# with 128-row tiles: first call large (split into 12 slices: ~25 MiB of partials), second smaller
# (16 slices of a 64 x 1000 output), then a shape that does not split; automatic: the thin kernel
CALLS = [(128, 4096, 4096), (64, 1000, 2000), (300, 520, 704)]
ENVS = {"auto": {}, "tile128": {"BSFP8_GEMM_TILE_M": "128"}, "forced3": {"BSFP8_GEMM_SPLIT": "3"}}


@pytest.mark.parametrize("env", list(ENVS), ids=list(ENVS))
def test_noalloc_matches_allocating_entry(env, monkeypatch):
    for k in ("BSFP8_GEMM_SPLIT", "BSFP8_GEMM_TILE_M", "BSFP8_GEMM_TILE_N"):
        monkeypatch.delenv(k, raising=False)
    for k, v in ENVS[env].items():
        monkeypatch.setenv(k, v)
    for i, (M, N, K) in enumerate(CALLS):
        print(f"noalloc call {i}: M={M} N={N} K={K} split={env}", flush=True)
        qa, sa, qw, sw, oqa, osa, oqw, osw = _operands(M, N, K, 40 + i)
        buf, c = _guarded(M, N)
        bf.gemm_1x128_128x128_noalloc(qa, sa, qw, sw, c)
        ref = bf.gemm_1x128_128x128(qa, sa, qw, sw)
        torch.cuda.synchronize()
        _check_guard(buf, M, N)
        got = c.float().cpu().numpy()
        assert np.array_equal(got, ref.float().cpu().numpy()), f"call {i} differs from the allocating entry"
        co = oracle.gemm_1x128_128x128(oqa, osa, oqw, osw, osw.shape[1], 1)
        rep = oracle.gemm_tolerance_report(got, co)
        assert rep["ok"], (i, rep)


def test_noalloc_rejects_a_plan_beyond_the_scratch(monkeypatch):
    """64 slices of a 512 x 1024 fp32 partial tile need 128 MiB, twice the scratch: the call
    returns BSFP8_ESCRATCH before launching anything and leaves C untouched."""
    M, N, K = 512, 1024, 8192
    monkeypatch.setenv("BSFP8_GEMM_SPLIT", "64")
    qa = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    qw = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    sa = torch.ones((K // 128, M), dtype=torch.float32, device=DEV)
    sw = torch.ones((N // 128, K // 128), dtype=torch.float32, device=DEV)
    c = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bf.Bsfp8Error) as e:
        bf.gemm_1x128_128x128_noalloc(qa, sa, qw, sw, c)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.all(c == 3.0)
