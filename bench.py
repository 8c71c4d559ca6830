"""Benchmark of the blockwise FP8 linear-layer hot path on one MI355X.

Step (the timed unit): the 4096^3 forward pass of a blockwise-FP8 linear layer,
    quantize_lhs(A [4096,4096]) + quantize_weight_128x128(W [4096,4096]) + gemm_1x128_128x128,
the two quantizations in one launch (quantize_lhs_and_weight: same outputs as the two calls),
on seeded synthetic bf16 inputs (A ~ N(0,1), W ~ N(0, 0.02^2)) already resident in HBM. Steps
rotate over several input/output buffer sets (> 1 GB in total) so the 256 MB last-level cache
does not serve the inputs of the next step.

Printed: one JSON line with the whole-step throughput (2MNK per step time, TFLOP/s), the GEMM's
roofline (TFLOP/s against the dense FP8 MFMA peak), the quantizers' GB/s against HBM, per-kernel
figures for every kernel of the path on the training-step and outlier shapes, and the CPU oracle
timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0   # MI355X dense f16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
BLOCK = 128


def _cdiv(a, b):
    return (a + b - 1) // b


def lhs_bytes(M, K):
    """Algorithmic bytes of a 1x128 / 128x1 activation quantizer: read 2 B, write 1 B per element,
    plus one fp32 scale per 128 elements."""
    return 2 * M * K + M * K + 4 * M * ((K + BLOCK - 1) // BLOCK)


def dual_bytes(R, C):
    """Algorithmic bytes of the one-pass 1x128 + 128x1 quantizer: read 2 B, write 2 B per element,
    plus the two scale tensors."""
    return 2 * R * C + 2 * R * C + 4 * R * ((C + BLOCK - 1) // BLOCK) + 4 * C * ((R + BLOCK - 1) // BLOCK)


def weight_bytes(N, K, with_qT):
    return 2 * N * K + N * K * (2 if with_qT else 1) + 4 * ((N + 127) // 128) * ((K + 127) // 128)


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence: recording it writes a timestamp
    without the system-scope cache writeback/invalidate a default event performs, so the kernels
    around it run as they would without the event (HIP documents the flag for timing)."""
    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._ctypes = ctypes
        self.h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.h, self._ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = self._ctypes.c_float()
        TimingEvent._hip.hipEventSynchronize(end.h)
        rc = TimingEvent._hip.hipEventElapsedTime(self._ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


def measured_traffic(kernel):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE record in profiles/, or None
    when the kernel source has changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    csrc = os.path.join(ROOT, "blockwise_scaled_fp8_act_amd", "csrc")
    h = hashlib.sha256()
    for f in ("gemm.hip", "device_common.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return rec.get("traffic_bytes")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=8, help="rotated buffer sets (cold cache)")
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="run the step for at least this long before the warm-up steps, so the "
                        "GPU clock has settled under sustained load")
    p.add_argument("--no-rows", action="store_true", help="omit the per-kernel shape table")
    p.add_argument("--no-cpu-baseline", action="store_true", help="omit the CPU oracle leg")
    p.add_argument("--cpu-rows", type=int, default=4096, help="GEMM rows in the CPU oracle sample")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES bytes 5 times (the reference "
                        "kernel for scaling HBM traffic counters) and exit")
    return p.parse_args()


def copy_probe(nbytes):
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reads": nbytes, "writes": nbytes}))


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   f"(got {args.gpus}); multi-GPU sharding is design only"}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        sys.exit(2)

    import torch
    import blockwise_scaled_fp8_act_amd as bf
    from blockwise_scaled_fp8_act_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dev_bf16(h):
        return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).to(dev)

    # ---------------------------------------------------------------- step workload
    d = inputs.make_workload(2)
    A_h, W_h = d["A"], d["W"]
    M, K = A_h.shape
    N = W_h.shape[0]
    Kb, Nb = K // BLOCK, N // BLOCK
    sets = []
    for i in range(args.sets):
        A = dev_bf16(A_h)
        W = dev_bf16(W_h)
        sets.append(dict(
            A=A, W=W,
            qa=torch.empty((M, K), dtype=torch.uint8, device=dev),
            sa=torch.empty((Kb, M), dtype=torch.float32, device=dev),
            qw=torch.empty((N, K), dtype=torch.uint8, device=dev),
            sw=torch.empty((Nb, Kb), dtype=torch.float32, device=dev),
            c=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        ))
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())

    def step(s, ev=None, per_kernel=False):
        # ev: events recorded on the launch stream; in the timed loop only the GEMM is bracketed
        # (its duration feeds the roofline), to keep event packets between kernels to a minimum
        if per_kernel:
            ev[0].record(stream)
        bf.quantize_lhs_and_weight(s["A"], s["W"], s["qa"], s["sa"], s["qw"], None, s["sw"],
                                   stream=stream)
        if ev is not None:
            ev[1].record(stream)
        bf.gemm_1x128_128x128(s["qa"], s["sa"], s["qw"], s["sw"], c=s["c"], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    # the chip's clock takes ~10-20 ms of sustained load to settle after an idle period (it dips
    # first, then rises: a 4096^3 GEMM launch takes ~79 us in the first few ms and ~63 us once
    # settled), so the steps run for at least --settle-ms before the W counted warm-up steps
    evs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]
    t_start = TimingEvent()
    t_end = TimingEvent()
    settle(lambda i: step(sets[i % len(sets)]), args.settle_ms, torch)
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    # the GEMM of every EVERY-th step is bracketed by an event pair (each pair costs ~1 us of
    # stream time, so not every step carries one)
    EVERY = 5
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i] if i % EVERY == 0 else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    gemm_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(0, args.steps, EVERY)])

    # per-kernel duration of the quantizer launch: a separate pass of the same steps with every
    # kernel bracketed (not part of the timed region)
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i], per_kernel=True)
    torch.cuda.synchronize()
    k_ms = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(2)] for e in evs])
    k_avg = k_ms.mean(axis=0)
    k_med = np.median(k_ms, axis=0)
    k_avg[1], k_med[1] = gemm_ms.mean(), np.median(gemm_ms)  # the GEMM figures are the timed region's

    # the quantizer launch's own duration: the step's quantizer launched back to back over the
    # rotating sets, one event pair per batch (an event pair around a single launch also spans its
    # dispatch, as the in-step figure above does)
    q_batch_ms, q_p10, q_p90 = _time_kernel(
        lambda i: bf.quantize_lhs_and_weight(sets[i % len(sets)]["A"], sets[i % len(sets)]["W"],
                                             sets[i % len(sets)]["qa"], sets[i % len(sets)]["sa"],
                                             sets[i % len(sets)]["qw"], None, sets[i % len(sets)]["sw"],
                                             stream=stream), args.steps, stream, torch)

    flops = 2.0 * M * N * K
    gemm_tflops = flops / (k_avg[1] * 1e-3) / 1e12
    q_bytes = lhs_bytes(M, K) + weight_bytes(N, K, False)
    q_gbs = q_bytes / (q_batch_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- per-kernel shape table
    rows = []
    if not args.no_rows:
        rows = kernel_rows(bf, inputs, dev_bf16, dev, stream, torch)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        s0 = sets[0]
        gpu = {k: s0[k].cpu().numpy() for k in ("qa", "sa", "qw", "sw")}
        gpu["c"] = s0["c"].float().cpu().numpy()
        cpu = cpu_baseline(A_h, W_h, args.cpu_rows, gpu)

    out = {
        "metric": "blockwise-FP8 GEMM TFLOPS @4096^3 (% FP8 MFMA peak) + quantizer GB/s (% HBM)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn",
        "data": "synthetic (seeded numpy PCG64, bf16 RNE)",
        "config": {
            "workload": "forward 4096^3: quantize_lhs A[4096,4096] + quantize_weight_128x128 "
                        "W[4096,4096] (one launch) + gemm_1x128_128x128 (A~N(0,1), W~N(0,0.02^2))",
            "M": M, "N": N, "K": K, "rotated_sets": len(sets),
            "arithmetic": "bf16 in; float8_e4m3fn codes with fp32 scales; fp8 x fp8 matrix-core "
                          "products, fp32 per-K-block rescale and accumulation; bf16 out",
            "rotated_bytes": set_bytes * len(sets),
        },
        "roofline": {
            "kernel": "gemm_1x128_128x128",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": measured_traffic("gemm_1x128_128x128"),
            "traffic_unit": "bytes per launch (HBM/MALL, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
        },
        "step_kernels": {
            "quantize_lhs_and_weight": {"avg_us": round(q_batch_ms * 1e3, 2),
                                        "p10_us": round(q_p10 * 1e3, 2),
                                        "p90_us": round(q_p90 * 1e3, 2),
                                        "in_step_avg_us": round(k_avg[0] * 1e3, 2),
                                        "in_step_median_us": round(k_med[0] * 1e3, 2),
                                        "GB/s": round(q_gbs, 1),
                                        "frac_hbm": round(q_gbs / PEAK_HBM_GBS, 4)},
            "gemm_1x128_128x128": {"avg_us": round(k_avg[1] * 1e3, 2),
                                   "median_us": round(k_med[1] * 1e3, 2),
                                   "p10_us": round(float(np.percentile(gemm_ms, 10)) * 1e3, 2),
                                   "p90_us": round(float(np.percentile(gemm_ms, 90)) * 1e3, 2),
                                   "TFLOP/s": round(gemm_tflops, 1),
                                   "frac_mfma": round(gemm_tflops / PEAK_FP8_TFLOPS, 4)},
        },
        "rows": rows,
        "cpu_baseline": cpu,
        "context": {"pages_mi300x_triton_fp8_tflops_4096": 299.3,
                    "pages_mi300x_hipblas_bf16_tflops_4096": 565.8},
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out))


def settle(fn, min_ms, torch, chunk=50):
    """Run fn(0), fn(1), ... until at least min_ms of wall time has passed (synchronizing every
    `chunk` calls), so the GPU's clock has settled under sustained load before timing starts."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(chunk):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return i


SETTLE_ROW_MS = 30.0


def _time_kernel(fn, reps, stream, torch, batches=8):
    """Duration (ms) of fn(i) over reps back-to-back launches, as (average, p10, p90): the launches
    run in `batches` consecutive batches, each bracketed by HIP events on `stream` (so host-side
    launch cost never shows as GPU time); the average is over all launches, p10 and p90 over the
    batches' per-launch averages. The launches first run for SETTLE_ROW_MS so the clock has
    settled after the host-side set-up."""
    settle(fn, SETTLE_ROW_MS, torch, chunk=10)
    per = max(1, reps // batches)
    ev = [TimingEvent() for _ in range(batches + 1)]
    i = 0
    ev[0].record(stream)
    for b in range(batches):
        for _ in range(per):
            fn(i)
            i += 1
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[b].elapsed_time(ev[b + 1]) / per for b in range(batches)])
    return float(ms.mean()), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def _time_graph(fn, per, torch, batches=8):
    """Duration (ms) per launch of fn(i), i = 0 .. per-1, recorded once into a HIP graph (every
    call on torch's current stream, which is the capture stream inside the capture) and replayed
    `batches` times, each replay bracketed by HIP events: (average, p10, p90) over the replays. A
    replay starts its kernels back to back, so the host's per-call cost does not show, as it does for
    launches from Python when one kernel takes less time than one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per):
            fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    settle(lambda i: graph.replay(), SETTLE_ROW_MS, torch, chunk=2)
    ev = [TimingEvent() for _ in range(batches + 1)]
    ev[0].record(stream)
    for b in range(batches):
        graph.replay()
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[b].elapsed_time(ev[b + 1]) / per for b in range(batches)])
    del graph
    return float(ms.mean()), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def kernel_rows(bf, inputs, dev_bf16, dev, stream, torch, reps=32, nsets=4):
    """Per-kernel timings on the training-step (8192 tokens, 4096x4096 weight) and outlier
    (16384 x 5120 x 5120) shapes, each rotating over buffer sets larger than the cache."""
    out = []

    def add(name, shape, t, work, unit, peak=None, **extra):
        avg, p10, p90 = t
        rate = work / (avg * 1e-3)
        if unit == "GB/s":
            r, peak = rate / 1e9, peak or PEAK_HBM_GBS
        else:
            r, peak = rate / 1e12, peak or PEAK_FP8_TFLOPS
        out.append({"kernel": name, "shape": shape, "avg_us": round(avg * 1e3, 2),
                    "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2), unit: round(r, 1),
                    "frac": round(r / peak, 4), **extra})

    d3 = inputs.make_workload(3)
    T, D = d3["X"].shape
    X = [dev_bf16(d3["X"]) for _ in range(nsets)]
    dY = [dev_bf16(d3["dY"]) for _ in range(nsets)]
    W = [dev_bf16(d3["W"]) for _ in range(nsets)]
    Kb = D // BLOCK
    qx = [torch.empty((T, D), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sx = [torch.empty((Kb, T), dtype=torch.float32, device=dev) for _ in range(nsets)]
    qxT = [torch.empty((D, T), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sxT = [torch.empty((T // BLOCK, D), dtype=torch.float32, device=dev) for _ in range(nsets)]
    qdy = [torch.empty((T, D), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sdy = [torch.empty((Kb, T), dtype=torch.float32, device=dev) for _ in range(nsets)]
    qdyT = [torch.empty((D, T), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sdyT = [torch.empty((T // BLOCK, D), dtype=torch.float32, device=dev) for _ in range(nsets)]
    qw = [torch.empty((D, D), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    qwT = [torch.empty((D, D), dtype=torch.uint8, device=dev) for _ in range(nsets)]
    sw = [torch.empty((Kb, Kb), dtype=torch.float32, device=dev) for _ in range(nsets)]
    out_c = [torch.empty((T, D), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    dw = [torch.empty((D, D), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]

    j = lambda i: i % nsets  # noqa: E731
    a = _time_kernel(lambda i: bf.quantize_lhs(X[j(i)], qx[j(i)], sx[j(i)], stream=stream), reps, stream, torch)
    add("quantize_lhs", [T, D], a, lhs_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_lhs(dY[j(i)], qdy[j(i)], sdy[j(i)], stream=stream), reps, stream, torch)
    add("quantize_lhs(dY)", [T, D], a, lhs_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_rhs(X[j(i)], qxT[j(i)], sxT[j(i)], stream=stream), reps, stream, torch)
    add("quantize_rhs", [T, D], a, lhs_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_rhs(dY[j(i)], qdyT[j(i)], sdyT[j(i)], stream=stream), reps, stream, torch)
    add("quantize_rhs(dY)", [T, D], a, lhs_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_lhs_and_rhs(X[j(i)], qx[j(i)], sx[j(i)], qxT[j(i)], sxT[j(i)],
                                                      stream=stream), reps, stream, torch)
    add("quantize_lhs_and_rhs", [T, D], a, dual_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_lhs_and_rhs(dY[j(i)], qdy[j(i)], sdy[j(i)], qdyT[j(i)], sdyT[j(i)],
                                                      stream=stream), reps, stream, torch)
    add("quantize_lhs_and_rhs(dY)", [T, D], a, dual_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_weight_128x128(W[j(i)], qw[j(i)], qwT[j(i)], sw[j(i)], stream=stream),
                        reps, stream, torch)
    add("quantize_weight_128x128(+qT)", [D, D], a, weight_bytes(D, D, True), "GB/s")
    fl = 2.0 * T * D * D
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qx[j(i)], sx[j(i)], qw[j(i)], sw[j(i)], c=out_c[j(i)],
                                                        stream=stream), reps, stream, torch)
    add("gemm_1x128_128x128 fwd", [T, D, D], a, fl, "TFLOP/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qdy[j(i)], sdy[j(i)], qwT[j(i)], sw[j(i)], 1, Kb,
                                                        c=out_c[j(i)], stream=stream), reps, stream, torch)
    add("gemm_1x128_128x128 dgrad", [T, D, D], a, fl, "TFLOP/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x1(qdyT[j(i)], sdyT[j(i)], qxT[j(i)], sxT[j(i)], c=dw[j(i)],
                                                      stream=stream), reps, stream, torch)
    add("gemm_1x128_128x1 wgrad", [D, D, T], a, fl, "TFLOP/s")
    # the whole training step of one linear layer through torch.autograd (quantize X, W, dY; the
    # forward, dgrad and wgrad GEMMs), 3 GEMMs of 2*T*D*D flop each
    Xg = [x.view(torch.bfloat16).clone().requires_grad_(True) for x in X[:2]]
    Wg = [w.view(torch.bfloat16).clone().requires_grad_(True) for w in W[:2]]
    dYg = [y.view(torch.bfloat16) for y in dY[:2]]

    def train_step(i):
        k = i % 2
        Xg[k].grad = None
        Wg[k].grad = None
        bf.blockwise_fp8_linear(Xg[k], Wg[k]).backward(dYg[k])

    a = _time_kernel(train_step, reps, stream, torch)
    add("linear fwd+dgrad+wgrad (autograd, all quantizers)", [T, D, D], a, 3 * fl, "TFLOP/s")

    # token counts off the 128 grid: the last K-block is partial (8000 tokens: wgrad K = 8000;
    # forward with 4000 input features)
    Tr, Kr = 8000, 4000
    a = _time_kernel(lambda i: bf.gemm_1x128_128x1(qdyT[j(i)][:, :Tr], sdyT[j(i)][:_cdiv(Tr, BLOCK)],
                                                      qxT[j(i)][:, :Tr], sxT[j(i)][:_cdiv(Tr, BLOCK)],
                                                      c=dw[j(i)], K=Tr, stream=stream), reps, stream, torch)
    add("gemm_1x128_128x1 wgrad, 8000 tokens (partial last K-block)", [D, D, Tr], a, 2.0 * D * D * Tr,
        "TFLOP/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qx[j(i)][:, :Kr], sx[j(i)][:_cdiv(Kr, BLOCK)],
                                                        qw[j(i)][:, :Kr], sw[j(i)], Kb, 1, c=out_c[j(i)],
                                                        K=Kr, stream=stream), reps, stream, torch)
    add("gemm_1x128_128x128 fwd, K = 4000 (partial last K-block)", [T, D, Kr], a, 2.0 * T * D * Kr,
        "TFLOP/s")

    # float8_e4m3fnuz (FP8_MAX 240): the same quantizers; the GEMMs widen the codes to f16 and run
    # on the f16 matrix instructions, so their peak is the dense f16 one
    fz = "e4m3fnuz"
    a = _time_kernel(lambda i: bf.quantize_lhs_and_rhs(X[j(i)], qx[j(i)], sx[j(i)], qxT[j(i)], sxT[j(i)],
                                                      stream=stream, fmt=fz), reps, stream, torch)
    add("quantize_lhs_and_rhs e4m3fnuz", [T, D], a, dual_bytes(T, D), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_weight_128x128(W[j(i)], qw[j(i)], qwT[j(i)], sw[j(i)], stream=stream,
                                                             fmt=fz), reps, stream, torch)
    add("quantize_weight_128x128(+qT) e4m3fnuz", [D, D], a, weight_bytes(D, D, True), "GB/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qx[j(i)], sx[j(i)], qw[j(i)], sw[j(i)], c=out_c[j(i)],
                                                        stream=stream, fmt=fz), reps, stream, torch)
    add("gemm_1x128_128x128 fwd e4m3fnuz (f16 MFMA)", [T, D, D], a, fl, "TFLOP/s", PEAK_F16_TFLOPS)
    a = _time_kernel(lambda i: bf.gemm_1x128_128x1(qdyT[j(i)], sdyT[j(i)], qxT[j(i)], sxT[j(i)], c=dw[j(i)],
                                                      stream=stream, fmt=fz), reps, stream, torch)
    add("gemm_1x128_128x1 wgrad e4m3fnuz (f16 MFMA)", [D, D, T], a, fl, "TFLOP/s", PEAK_F16_TFLOPS)
    del X, dY, W, qx, sx, qxT, sxT, qdy, sdy, qdyT, sdyT, qw, qwT, sw, out_c, dw, Xg, Wg, dYg
    torch.cuda.empty_cache()

    # expert-grouped (MoE) GEMMs: 8 experts, 16384 routed tokens split unevenly in multiples of
    # 128, 4096 -> 2048 features per expert; forward (rows grouped) and weight gradient (tokens
    # grouped), 2*T*2048*4096 flop each
    E, Tm, Di, Do = 8, 16384, 4096, 2048
    gm = np.random.Generator(np.random.PCG64(5))
    counts = gm.multinomial(Tm // BLOCK, np.full(E, 1.0 / E)) * BLOCK
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int64, device=dev)
    nsm = 2
    Am = [dev_bf16(inputs.normal_bf16(gm, (Tm, Di))) for _ in range(nsm)]
    Wm = dev_bf16(inputs.normal_bf16(gm, (E * Do, Di), 0.02))
    dYm = dev_bf16(inputs.normal_bf16(gm, (Tm, Do), 0.01))
    qam = [bf.quantize_lhs(x) for x in Am]
    qwm, _, swm = bf.quantize_weight_128x128(Wm, want_qT=False)
    qxTm, sxTm = bf.quantize_rhs(Am[0])
    qdyTm, sdyTm = bf.quantize_rhs(dYm)
    cm = [torch.empty((Tm, Do), dtype=torch.bfloat16, device=dev) for _ in range(nsm)]
    dwm = torch.empty((E, Do, Di), dtype=torch.bfloat16, device=dev)
    Kbm, Nbm = Di // BLOCK, Do // BLOCK
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128_grouped(
        qam[i % nsm][0], qam[i % nsm][1], qwm, swm, offs, E, b_stride=Do * Di, bs_stride=Nbm * Kbm,
        bs_stride_nb=Kbm, bs_stride_kb=1, c=cm[i % nsm], N=Do, stream=stream), reps, stream, torch)
    add("gemm_1x128_128x128_grouped fwd (8 experts)", [Tm, Do, Di], a, 2.0 * Tm * Do * Di, "TFLOP/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x1_grouped(qdyTm, sdyTm, qxTm, sxTm, offs, E, c=dwm,
                                                           stream=stream), reps, stream, torch)
    add("gemm_1x128_128x1_grouped wgrad (8 experts)", [Do, Di, Tm], a, 2.0 * Tm * Do * Di, "TFLOP/s")
    # ragged routing: token counts drawn per token, not in multiples of 128; the expert-grouped
    # 128x1 quantizer writes the 128-padded layout the grouped weight gradient reads
    counts_r = gm.multinomial(Tm, np.full(E, 1.0 / E))
    offs_r = torch.tensor(np.concatenate([[0], np.cumsum(counts_r)]), dtype=torch.int64, device=dev)
    Gr = _cdiv(Tm, BLOCK) + E
    qTr = [torch.empty((Di, Gr * BLOCK), dtype=torch.uint8, device=dev) for _ in range(nsm)]
    sr = [torch.empty((Gr, Di), dtype=torch.float32, device=dev) for _ in range(nsm)]
    pr = torch.empty(E + 1, dtype=torch.int64, device=dev)
    a = _time_kernel(lambda i: bf.quantize_rhs_grouped(Am[i % nsm], offs_r, E, qT=qTr[i % nsm], s=sr[i % nsm],
                                                       padded_offsets=pr, stream=stream), reps, stream, torch)
    torch.cuda.synchronize()
    ptot = int(pr[-1].item())
    add("quantize_rhs_grouped (8 experts, ragged counts)", [Tm, Di], a,
        2 * Tm * Di + ptot * Di + 4 * (ptot // BLOCK) * Di, "GB/s")
    del qTr, sr, pr
    del Am, Wm, dYm, qam, qwm, swm, qxTm, sxTm, qdyTm, sdyTm, cm, dwm
    torch.cuda.empty_cache()

    # tail-masking workload (130 x 5120 x 1280): a few MB of data in 64 x 32 tiles of the thin kernel
    # (480 workgroups), served from cache; reported for completeness (its quantizers finish faster
    # than one launch from Python, so timing them here would time the host)
    d1 = inputs.make_workload(1)
    A1, W1 = dev_bf16(d1["A"]), dev_bf16(d1["W"])
    M1 = d1["A"].shape[0]
    N1, K1 = d1["W"].shape
    qa1, sa1 = bf.quantize_lhs(A1, stream=stream)
    qw1, _, sw1 = bf.quantize_weight_128x128(W1, want_qT=False, stream=stream)
    c1 = torch.empty((M1, N1), dtype=torch.bfloat16, device=dev)
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qa1, sa1, qw1, sw1, c=c1, stream=stream), reps,
                     stream, torch)
    gph = _time_graph(lambda i: bf.gemm_1x128_128x128_noalloc(qa1, sa1, qw1, sw1, c1), 16, torch)
    add("gemm_1x128_128x128 tail (warm cache)", [M1, N1, K1], a, 2.0 * M1 * N1 * K1, "TFLOP/s",
        graph_avg_us=round(gph[0] * 1e3, 2), graph_p10_us=round(gph[1] * 1e3, 2), graph_p90_us=round(gph[2] * 1e3, 2))
    del A1, W1, qa1, sa1, qw1, sw1, c1

    d4 = inputs.make_workload(4)
    M4, K4 = d4["A"].shape
    N4 = d4["W"].shape[0]
    ns4 = 3
    A4 = [dev_bf16(d4["A"]) for _ in range(ns4)]
    W4 = [dev_bf16(d4["W"]) for _ in range(ns4)]
    qa4 = [torch.empty((M4, K4), dtype=torch.uint8, device=dev) for _ in range(ns4)]
    sa4 = [torch.empty((K4 // BLOCK, M4), dtype=torch.float32, device=dev) for _ in range(ns4)]
    qw4 = [torch.empty((N4, K4), dtype=torch.uint8, device=dev) for _ in range(ns4)]
    sw4 = [torch.empty((N4 // BLOCK, K4 // BLOCK), dtype=torch.float32, device=dev) for _ in range(ns4)]
    c4 = [torch.empty((M4, N4), dtype=torch.bfloat16, device=dev) for _ in range(ns4)]
    k = lambda i: i % ns4  # noqa: E731
    a = _time_kernel(lambda i: bf.quantize_lhs(A4[k(i)], qa4[k(i)], sa4[k(i)], stream=stream), reps, stream, torch)
    add("quantize_lhs outlier", [M4, K4], a, lhs_bytes(M4, K4), "GB/s")
    a = _time_kernel(lambda i: bf.quantize_weight_128x128(W4[k(i)], qw4[k(i)], None, sw4[k(i)], want_qT=False,
                                                             stream=stream), reps, stream, torch)
    add("quantize_weight_128x128 outlier", [N4, K4], a, weight_bytes(N4, K4, False), "GB/s")
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qa4[k(i)], sa4[k(i)], qw4[k(i)], sw4[k(i)], c=c4[k(i)],
                                                        stream=stream), reps, stream, torch)
    add("gemm_1x128_128x128 outlier", [M4, N4, K4], a, 2.0 * M4 * N4 * K4, "TFLOP/s")
    del A4, W4, qa4, sa4, qw4, sw4, c4
    torch.cuda.empty_cache()

    # the forward GEMM at every shape of the ROCm page's performance table (its FP8 Triton GEMM on
    # MI300X, printed there as context: another chip, not a target). Operands from N(0,1) / N(0,
    # 0.02^2) bf16 through the quantizers, copied into enough rotating sets to exceed the 256 MB
    # last-level cache (at most 32 sets); shapes with few rows take the thin kernel's 64-row tiles.
    g8 = np.random.Generator(np.random.PCG64(8))
    for (Mp, Np, Kp, page_tflops) in PAGES_GEMM_TABLE:
        ap = dev_bf16(inputs.normal_bf16(g8, (Mp, Kp)))
        wp = dev_bf16(inputs.normal_bf16(g8, (Np, Kp), 0.02))
        qa0, sa0 = bf.quantize_lhs(ap)
        qw0, _, sw0 = bf.quantize_weight_128x128(wp, want_qT=False)
        del ap, wp
        per_set = Mp * Kp + Np * Kp + 4 * (sa0.numel() + sw0.numel()) + 2 * Mp * Np
        nsp = int(min(32, max(2, _cdiv(300 << 20, per_set))))
        ops = [(qa0.clone(), sa0.clone(), qw0.clone(), sw0.clone(),
                torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)) for _ in range(nsp)]
        del qa0, sa0, qw0, sw0
        a = _time_kernel(lambda i: bf.gemm_1x128_128x128(*ops[i % nsp][:4], c=ops[i % nsp][4], stream=stream),
                         reps, stream, torch)
        # the same launches replayed from a HIP graph (the allocation-free entry point, same
        # kernels and schedule): GPU time without the host's per-call cost
        gph = _time_graph(lambda i: bf.gemm_1x128_128x128_noalloc(*ops[i % nsp][:4], ops[i % nsp][4]),
                          2 * nsp, torch)
        fl = 2.0 * Mp * Np * Kp
        add(f"gemm_1x128_128x128 {Mp}x{Np}x{Kp} (pages' table shape)", [Mp, Np, Kp], a, fl, "TFLOP/s",
            pages_mi300x_fp8_tflops=page_tflops, rotated_sets=nsp,
            graph_avg_us=round(gph[0] * 1e3, 2), graph_p10_us=round(gph[1] * 1e3, 2),
            graph_p90_us=round(gph[2] * 1e3, 2), **{"graph_TFLOP/s": round(fl / (gph[0] * 1e-3) / 1e12, 1)})
        del ops
        torch.cuda.empty_cache()

    # the smallest workload (2 x 512 x 128: one K-block, 16 thin tiles): host-launch-bound, so it
    # is timed like the others but only shows the launch floor
    d0 = inputs.make_workload(0)
    A0, W0 = dev_bf16(d0["A"]), dev_bf16(d0["W"])
    qa_0, sa_0, qw_0, _, sw_0 = bf.quantize_lhs_and_weight(A0, W0)
    c0 = torch.empty((A0.shape[0], W0.shape[0]), dtype=torch.bfloat16, device=dev)
    a = _time_kernel(lambda i: bf.gemm_1x128_128x128(qa_0, sa_0, qw_0, sw_0, c=c0, stream=stream), reps,
                     stream, torch)
    gph = _time_graph(lambda i: bf.gemm_1x128_128x128_noalloc(qa_0, sa_0, qw_0, sw_0, c0), 16, torch)
    add("gemm_1x128_128x128 2x512x128 (launch floor)", [2, 512, 128], a, 2.0 * 2 * 512 * 128, "TFLOP/s",
        graph_avg_us=round(gph[0] * 1e3, 2), graph_p10_us=round(gph[1] * 1e3, 2), graph_p90_us=round(gph[2] * 1e3, 2))
    del A0, W0, qa_0, sa_0, qw_0, sw_0, c0
    return out


# The ROCm page's GEMM performance table: M, N, K and its FP8 Triton TFLOP/s on MI300X.
PAGES_GEMM_TABLE = [
    (128, 4096, 4096, 54.6), (512, 4096, 4096, 220.3), (2048, 4096, 4096, 294.1),
    (4096, 4096, 4096, 299.3), (8192, 4096, 4096, 306.2), (2048, 8192, 4096, 453.4),
    (4096, 8192, 4096, 470.5), (4096, 5120, 5120, 525.0),
]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(A_h, W_h, gemm_rows, gpu):
    """The CPU oracle (as it stands) on a bounded sample of the step: both quantizers on the full
    tensors, the GEMM on `gemm_rows` evenly spaced rows; scaled to the whole step. The same leg
    checks the GPU step's outputs (`gpu`: host copies of one set's codes, scales and C) against
    what the oracle computed: the codes and scales bit for bit, the sampled rows of C within the
    GEMM tolerance, and the SQNR of both against the fp64 product of the bf16 inputs. It also times
    the two quantizers on one thread."""
    import oracle
    M, K = A_h.shape
    N = W_h.shape[0]
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    qa, sa = oracle.quantize_lhs(A_h)
    qw, _, sw = oracle.quantize_weight_128x128(W_h, want_qT=False)
    t1 = time.perf_counter()
    rows = np.linspace(0, M - 1, gemm_rows).astype(np.int64)
    c_or = oracle.gemm_1x128_128x128(qa, sa, qw, sw, sw.shape[1], 1, rows=rows)
    t2 = time.perf_counter()
    step_s = (t1 - t0) + (t2 - t1) * (M / gemm_rows)

    # one thread: the quantizers over the same tensors
    oracle.set_num_threads(1)
    try:
        t3 = time.perf_counter()
        oracle.quantize_lhs(A_h)
        oracle.quantize_weight_128x128(W_h, want_qT=False)
        q1_s = time.perf_counter() - t3
    finally:
        oracle.set_num_threads(threads)
    q_bytes = lhs_bytes(M, K) + weight_bytes(N, K, False)

    parity = None
    if gpu is not None:
        quant_exact = bool(np.array_equal(gpu["qa"], qa) and np.array_equal(gpu["sa"].view(np.uint32), sa.view(np.uint32))
                           and np.array_equal(gpu["qw"], qw) and np.array_equal(gpu["sw"].view(np.uint32), sw.view(np.uint32)))
        c_gpu = gpu["c"][rows]
        rep = oracle.gemm_tolerance_report(c_gpu, c_or)
        ref = oracle.matmul_bf16_f64(A_h, W_h, rows=rows)
        parity = {
            "quantizers_bit_exact": quant_exact,
            "gemm_rows_checked": int(rows.size),
            "gemm_within_tolerance": rep["ok"],
            "gemm_rel_frobenius": rep["rel_frobenius"],
            "sqnr_gpu_db": round(oracle.sqnr_db(ref, c_gpu), 3),
            "sqnr_oracle_db": round(oracle.sqnr_db(ref, c_or), 3),
            "verdict": "pass" if quant_exact and rep["ok"] else "FAIL",
        }
    return {
        "value": round(2.0 * M * N * K / step_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"quantize_lhs + quantize_weight_128x128 on the full 4096x4096 tensors, GEMM on "
                  f"{gemm_rows} of {M} rows; GEMM time scaled by {M / gemm_rows:g}",
        "measured_s": round(t2 - t0, 2),
        "quant_s": round(t1 - t0, 3),
        "gemm_sample_s": round(t2 - t1, 3),
        "quant_1thread_s": round(q1_s, 3),
        "quant_1thread_GB/s": round(q_bytes / q1_s / 1e9, 3),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
        "cpu_model": _cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count(),
        "parity": parity,
    }


if __name__ == "__main__":
    main()
