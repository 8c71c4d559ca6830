"""gemm_1x128_128x128_noalloc under HIP graph capture: the allocation-free entry point is for
callers that record their launches into a graph. Three calls (a K split whose partial tiles live in
the static scratch, a 128-row-tile shape and a 256-row-tile shape) are captured once and the graph
is replayed several times, with other eager work on the GPU between the replays; every replay must
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


def test_noalloc_gemm_graph_replays_match_eager(monkeypatch):
    monkeypatch.delenv("BSFP8_GEMM_SPLIT", raising=False)
    monkeypatch.delenv("BSFP8_GEMM_TILE_M", raising=False)
    shapes = [(128, 4096, 4096), (300, 520, 704), (1024, 2048, 1024)]
    ops = [_operands(M, N, K, 60 + i) for i, (M, N, K) in enumerate(shapes)]
    eager = []
    for (M, N, K), o in zip(shapes, ops):
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        bf.gemm_1x128_128x128_noalloc(*o, c)
        eager.append(c)
    torch.cuda.synchronize()
    eager = [c.clone() for c in eager]

    outs = [torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") for (M, N, K) in shapes]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside the capture
        for o, c in zip(ops, outs):
            bf.gemm_1x128_128x128_noalloc(*o, c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for o, c in zip(ops, outs):
            bf.gemm_1x128_128x128_noalloc(*o, c)
    torch.cuda.synchronize()

    junk = torch.randn(1 << 22, device="cuda")
    for r in range(4):
        for c in outs:
            c.fill_(float("nan"))
        # eager work between replays, including a library GEMM that uses the same scratch
        junk.mul_(1.0001)
        other = torch.empty((64, 4096), dtype=torch.bfloat16, device="cuda")
        bf.gemm_1x128_128x128_noalloc(*_operands(64, 4096, 4096, 99), other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(outs, eager)):
            assert torch.equal(c.view(torch.int16), e.view(torch.int16)), f"replay {r}, call {i}"
