"""GPU parity of the expert-grouped (MoE) GEMMs against the oracle applied expert by expert.

Grouped forward / dgrad: expert e owns rows [offsets[e], offsets[e+1]) of A and C and its own
weight; per expert the result must be the dense gemm_1x128_128x128 of those rows (oracle in fp64,
GEMM tolerance). Rows outside every expert's range must keep their prefilled sentinel. Grouped
weight gradient: expert e contracts over its own token columns; per expert the dense
gemm_1x128_128x1 of that K range. The grouped kernels run on the oracle's codes and scales, so the
GEMM is checked in isolation (the quantizers have their own bit-exact tests).
"""
import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_act_amd as bf
import oracle
from blockwise_scaled_fp8_act_amd import inputs
from tests._gpu import DEV, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1  # a bf16 NaN pattern no GEMM output has


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _check(c_gpu, c_oracle, what):
    rep = oracle.gemm_tolerance_report(c_gpu, c_oracle)
    assert rep["ok"], f"{what}: {rep}"


def _bf16_of(c):
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def _stacked_weights(E, N, K, seed):
    w = inputs.normal_bf16(_g(seed), (E * N, K), 0.02)        # W [E, N, K] stacked as [E*N, K]
    q, qT, s = oracle.quantize_weight_128x128(w)              # blocks never straddle experts
    return w, q, qT, s


@pytest.mark.parametrize("offsets", [
    [5, 305, 305, 822, 1033],        # lead and tail rows outside every expert, an empty expert
    [0, 256, 512, 768, 1040],        # whole row tiles
    [0, 1040],                       # one expert
    [3, 600, 400, 900, 1040],        # a decreasing boundary: clamped to an empty expert
], ids=["ragged", "aligned", "single", "clamped"])
def test_grouped_forward_and_dgrad(offsets):
    E = len(offsets) - 1
    M, N, K = 1040, 256, 512
    Kb, Nb = K // 128, N // 128
    a = inputs.normal_bf16(_g(1), (M, K))
    dy = inputs.normal_bf16(_g(2), (M, N), 0.01)
    w, q, qT, s = _stacked_weights(E, N, K, seed=3)
    qa, sa = oracle.quantize_lhs(a)
    qdy, sdy = oracle.quantize_lhs(dy)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)

    # forward: B_e = rows e*N .. of q, scales s[e*Nb .., :] with strides (Kb, 1)
    c = torch.full((M, N), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    bf.gemm_1x128_128x128_grouped(to_dev(qa), to_dev(sa), to_dev(q), to_dev(s), off, E,
                                  b_stride=N * K, bs_stride=Nb * Kb, bs_stride_nb=Kb,
                                  bs_stride_kb=1, c=c, N=N)
    # dgrad: B_e = columns e*N .. of qT [K, E*N] (b_stride N bytes, ldb E*N), scales transposed
    dx = torch.full((M, K), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    bf.gemm_1x128_128x128_grouped(to_dev(qdy), to_dev(sdy), to_dev(qT), to_dev(s), off, E,
                                  b_stride=N, bs_stride=Nb * Kb, bs_stride_nb=1, bs_stride_kb=Kb,
                                  ldb=E * N, c=dx, N=K)
    torch.cuda.synchronize()

    c_h, dx_h = c.float().cpu().numpy(), dx.float().cpu().numpy()
    covered = np.zeros(M, dtype=bool)
    prev = 0
    for e in range(E):
        lo = min(max(offsets[e], prev), M)
        hi = min(max(offsets[e + 1], lo), M)
        prev = hi
        if hi == lo:
            continue
        covered[lo:hi] = True
        r = np.arange(lo, hi)
        qe = q[e * N:(e + 1) * N]
        se = s[e * Nb:(e + 1) * Nb]
        co = oracle.gemm_1x128_128x128(qa[r], sa[:, r], qe, se, Kb, 1)
        _check(c_h[r], co, f"forward expert {e}")
        qTe = np.ascontiguousarray(qT[:, e * N:(e + 1) * N])
        co = oracle.gemm_1x128_128x128(qdy[r], sdy[:, r], qTe, se, 1, Kb)
        _check(dx_h[r], co, f"dgrad expert {e}")
    assert np.all(_bf16_of(c)[~covered] == SENTINEL), "forward wrote a row outside every expert"
    assert np.all(_bf16_of(dx)[~covered] == SENTINEL), "dgrad wrote a row outside every expert"


def test_grouped_forward_at_the_workload():
    """The expert-grouped forward workload (8 experts, 16384 tokens in multiples of 128, 4096 ->
    2048; six experts end in a half-filled 256-row tile): sampled rows of every expert, its first and
    last rows and the rows around the last whole tile included, match the oracle."""
    E, T, Di, Do = 8, 16384, 4096, 2048
    counts = np.array([2432, 2432, 1920, 1664, 1280, 2048, 2176, 2432])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    g = _g(11)
    a = inputs.normal_bf16(g, (T, Di))
    qa, sa = bf.quantize_lhs(to_dev(a))
    w, q, qT, s = _stacked_weights(E, Do, Di, seed=12)
    Kb, Nb = Di // 128, Do // 128
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    c = bf.gemm_1x128_128x128_grouped(qa, sa, to_dev(q), to_dev(s), off, E, b_stride=Do * Di,
                                      bs_stride=Nb * Kb, bs_stride_nb=Kb, bs_stride_kb=1, N=Do)
    torch.cuda.synchronize()
    qa_h, sa_h = qa.cpu().numpy(), sa.cpu().numpy()
    c_h = c.float().cpu().numpy()
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        r = np.unique(np.concatenate([[lo, hi - 1, hi - 128, hi - 129], g.integers(lo, hi, 28)]))
        co = oracle.gemm_1x128_128x128(qa_h[r], sa_h[:, r], q[e * Do:(e + 1) * Do], s[e * Nb:(e + 1) * Nb], Kb, 1)
        _check(c_h[r], co, f"expert {e}")


def test_grouped_single_expert_equals_dense():
    """E = 1 over all rows is the dense kernel, bit for bit (a shape with enough output tiles that
    the dense GEMM does not split K)."""
    M, N, K = 4200, 2304, 640
    a = to_dev(inputs.normal_bf16(_g(5), (M, K)))
    w = to_dev(inputs.normal_bf16(_g(6), (N, K), 0.02))
    qa, sa = bf.quantize_lhs(a)
    qw, _, sw = bf.quantize_weight_128x128(w, want_qT=False)
    dense = bf.gemm_1x128_128x128(qa, sa, qw, sw)
    off = torch.tensor([0, M], dtype=torch.int64, device=DEV)
    grouped = bf.gemm_1x128_128x128_grouped(qa, sa, qw, sw, off, 1, b_stride=0, bs_stride=0,
                                            bs_stride_nb=sw.stride(0), bs_stride_kb=1, N=N)
    torch.cuda.synchronize()
    assert torch.equal(dense.view(torch.int16), grouped.view(torch.int16))


@pytest.mark.parametrize("counts", [[256, 0, 384, 128], [128] * 8, [1024]],
                         ids=["ragged", "eight", "single"])
def test_grouped_weight_gradient(counts):
    E = len(counts)
    T = sum(counts)
    n_out, n_in = 256, 384
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = inputs.normal_bf16(_g(7), (T, n_in))
    dy = inputs.normal_bf16(_g(8), (T, n_out), 0.01)
    qxT, sx = oracle.quantize_rhs(x)      # 128x1 over all tokens = per expert (boundaries % 128 == 0)
    qdyT, sdy = oracle.quantize_rhs(dy)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    dw = bf.gemm_1x128_128x1_grouped(to_dev(qdyT), to_dev(sdy), to_dev(qxT), to_dev(sx), off, E)
    torch.cuda.synchronize()
    dw_h = dw.float().cpu().numpy()
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            assert np.all(dw_h[e] == 0.0), f"expert {e} with no tokens must give dW = 0"
            continue
        kr = slice(lo, hi)
        kbr = slice(lo // 128, hi // 128)
        co = oracle.gemm_1x128_128x1(np.ascontiguousarray(qdyT[:, kr]), sdy[kbr],
                                     np.ascontiguousarray(qxT[:, kr]), sx[kbr])
        _check(dw_h[e], co, f"wgrad expert {e}")


# ------------------------------------------------------------------ ragged expert token counts

RAGGED = [[300, 0, 5, 700, 128, 1], [1], [129, 127], [0, 0, 640]]


@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz"])
@pytest.mark.parametrize("N", [200, 203])
@pytest.mark.parametrize("counts", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_quantize_rhs_grouped_bit_exact(counts, N, fmt):
    """Groups restarting at each expert's first token, in the 128-padded layout: codes, scales and
    padded offsets equal the oracle's (quantize_rhs applied expert by expert) bit for bit, in the
    written region; N = 203 takes the unvectorised loads."""
    E = len(counts)
    lead = 7                                             # tokens before the first expert
    offsets = np.concatenate([[lead], lead + np.cumsum(counts)]).astype(np.int64)
    T = int(offsets[-1]) + 3                             # and after the last
    x = inputs.normal_bf16(_g(31 + N), (T, N))
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    qT, s, P = bf.quantize_rhs_grouped(xd, off, E, fmt=fmt)
    torch.cuda.synchronize()
    oqT, os_, oP = oracle.quantize_rhs_grouped(x, offsets, fmt=fmt)
    assert np.array_equal(P.cpu().numpy(), oP)
    tot = int(oP[-1])
    assert np.array_equal(qT.cpu().numpy()[:, :tot], oqT[:, :tot])
    assert np.array_equal(s.cpu().numpy()[:tot // 128].view(np.uint32), os_[:tot // 128].view(np.uint32))


@pytest.mark.parametrize("counts", [[300, 0, 5, 700, 128, 1], [129, 127], [1000]],
                         ids=lambda c: "-".join(map(str, c)))
def test_grouped_weight_gradient_ragged_counts(counts):
    """The MoE weight gradient for any routing: both token operands through quantize_rhs_grouped,
    then gemm_1x128_128x1_grouped over the padded offsets; expert by expert against the oracle's
    dense gemm_1x128_128x1 of that expert's own tokens (quantize_rhs of its slice of dY and X)."""
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(offsets[-1])
    n_out, n_in = 256, 384
    x = inputs.normal_bf16(_g(41), (T, n_in))
    dy = inputs.normal_bf16(_g(42), (T, n_out), 0.01)
    off = torch.tensor(offsets, dtype=torch.int64, device=DEV)
    qdyT, sdy, P = bf.quantize_rhs_grouped(torch.from_numpy(dy.view(np.int16)).to(DEV), off, E)
    qxT, sx, P2 = bf.quantize_rhs_grouped(torch.from_numpy(x.view(np.int16)).to(DEV), off, E)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dw = bf.gemm_1x128_128x1_grouped(qdyT, sdy, qxT, sx, P, E, status=status)
    torch.cuda.synchronize()
    assert torch.equal(P, P2) and int(status.item()) == 0
    dw_h = dw.float().cpu().numpy()
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            assert np.all(dw_h[e] == 0.0)
            continue
        a_q, a_s = oracle.quantize_rhs(dy[lo:hi])
        b_q, b_s = oracle.quantize_rhs(x[lo:hi])
        _check(dw_h[e], oracle.gemm_1x128_128x1(a_q, a_s, b_q, b_s), f"wgrad expert {e}")


def test_grouped_weight_gradient_flags_unaligned_offsets():
    """Boundaries off the 128 grid are not rounded: the experts they touch get NaN outputs and the
    status flag is set; an aligned expert in the same launch is computed normally, and a launch
    with aligned boundaries leaves a fresh flag at 0."""
    T, n_out, n_in = 256, 128, 256
    x = inputs.normal_bf16(_g(51), (T, n_in))
    dy = inputs.normal_bf16(_g(52), (T, n_out), 0.01)
    qxT, sx = oracle.quantize_rhs(x)
    qdyT, sdy = oracle.quantize_rhs(dy)
    args = [to_dev(qdyT), to_dev(sdy), to_dev(qxT), to_dev(sx)]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    off = torch.tensor([0, 128, 200, 256], dtype=torch.int64, device=DEV)
    dw = bf.gemm_1x128_128x1_grouped(*args, off, 3, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    dw_h = dw.float().cpu().numpy()
    assert np.all(np.isnan(dw_h[1])) and np.all(np.isnan(dw_h[2]))
    co = oracle.gemm_1x128_128x1(np.ascontiguousarray(qdyT[:, :128]), sdy[:1],
                                 np.ascontiguousarray(qxT[:, :128]), sx[:1])
    _check(dw_h[0], co, "aligned expert next to unaligned ones")
    fresh = torch.zeros(1, dtype=torch.int32, device=DEV)
    bf.gemm_1x128_128x1_grouped(*args, torch.tensor([0, 128, 256], dtype=torch.int64, device=DEV), 2,
                                status=fresh)
    torch.cuda.synchronize()
    assert int(fresh.item()) == 0
