"""gemm_1x128_128x128_noalloc under HIP graph capture: the allocation-free entry point is for
callers that record their launches into a graph. Four calls (a K split whose partial tiles live in
the static scratch, a thin-kernel shape, a 128-row-tile shape and a 256-row-tile shape; the schedule
of each set through the environment, which each call reads) are captured once and the graph is
replayed several times, with other eager work on the GPU between the replays; every replay must
reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
from blockwise_scaled_fp8_act_amd import inputs
from tests._gpu import to_dev

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = inputs.rng(seed)
    qa, sa = bf.quantize_lhs(to_dev(inputs.normal_bf16(g, (M, K))))
    qw, _, sw = bf.quantize_weight_128x128(to_dev(inputs.normal_bf16(g, (N, K), 0.02)), want_qT=False)
    return qa, sa, qw, sw


def _schedule(monkeypatch, tile_m):
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    monkeypatch.delenv("BSFP8_GEMM_TILE_N", raising=False)
    if tile_m:
        monkeypatch.setenv("BSFP8_GEMM_TILE_M", str(tile_m))
    else:
        monkeypatch.delenv("BSFP8_GEMM_TILE_M", raising=False)


def test_noalloc_gemm_graph_replays_match_eager(monkeypatch):
    # (shape, forced tile height): 128 rows here splits K into 12 slices; automatic: thin kernel
    calls = [((128, 4096, 4096), 128), ((300, 520, 704), 0), ((1024, 2048, 1024), 128), ((1024, 2048, 1024), 256)]
    shapes = [sh for sh, _ in calls]
    ops = [_operands(M, N, K, 60 + i) for i, (M, N, K) in enumerate(shapes)]

    def run_all(outs):
        for (_, tile_m), o, c in zip(calls, ops, outs):
            _schedule(monkeypatch, tile_m)
            bf.gemm_1x128_128x128_noalloc(*o, c)

    eager = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for (M, N, K) in shapes]
    run_all(eager)
    torch.cuda.synchronize()
    eager = [c.clone() for c in eager]

    outs = [torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") for (M, N, K) in shapes]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        run_all(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all(outs)
    torch.cuda.synchronize()

    junk = torch.randn(1 << 22, device="cuda")
    for r in range(4):
        for c in outs:
            c.fill_(float("nan"))
        # eager work between replays, including a library GEMM that uses the same scratch
        junk.mul_(1.0001)
        other = torch.empty((64, 4096), dtype=torch.bfloat16, device="cuda")
        _schedule(monkeypatch, 128)
        bf.gemm_1x128_128x128_noalloc(*_operands(64, 4096, 4096, 99), other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(outs, eager)):
            assert torch.equal(c.view(torch.int16), e.view(torch.int16)), f"replay {r}, call {i}"
