#!/usr/bin/env python3
"""Benchmark of the trellis dequantize-and-multiply hot path on one MI355X.

Headline: the axis-1 trellis GEMV of the Qwen MLP up projection, in 5120 ->
out 17408, T 256, L 12, k 2, M 1, bf16 activations, f32 scales, a 4096-entry
f32 codebook, seeded uniform random u32 codes. One step is one GEMV call
(codebook staging, code streaming, window decode, codebook gather, scale +
bf16 rounding, MFMA dot, reduction, bf16 store). The value is the effective
HBM bandwidth on packed-code bytes.

Every workload of the five configurations is timed the same way and reported
in the same JSON line under "workloads":
  C1 tiny GEMV 512 -> 256, k 2;
  C2 GEMV 5120 -> 17408, k 2 / 3 / 4 (k 2 is the headline);
  C3 scatter GEMV 17408 -> 5120 (axis 0), k 3, split-K partials + reduce;
  C4 prefill 5120 -> 17408, k 2 / 3 / 4 x M 5 / 8 / 16 / 32 (with the MFMA fraction);
  C5 MLP gate + up (one launch) + down, k 4, M 1 and 32; and the chained layer,
     gate + up with the fused SwiGLU epilogue feeding down.
Beside them, the decode ceiling: the random LDS gather rate of the kernels'
three table layouts, measured live by the probe kernel (trellis_probe.h).

Inputs are resident in HBM before timing starts. Calls rotate over enough
distinct code sets (>= 2 x 256 MB) that the 256 MB Infinity Cache cannot hold
them (C1 excepted: its 32 KB of codes make it launch-bound). The stored matrix
is 17408 x 5120 for every projection of C2-C5, so one pool of rotating code
sets per k serves the GEMV, the scatter (read as axis 0), the prefill and the
MLP's three projections.

Timing of each workload: a fixed clock-settling period of untimed calls
(SETTLE_S of wall time, independent of --warmup), then the W warm-up calls,
then a device synchronisation; LEAD untimed lead-in calls are enqueued so the
GPU is busy when the start event is recorded, then HIP events (on the stream
the kernels run on: torch's current stream, which the binding passes to the C
ABI) bracket exactly K back-to-back calls, followed by a synchronisation. So
the window holds the K calls' GPU time and no host launch latency. Five more
windows of K calls give the spread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra] [--no-cpu]
                       [--only NAME,...] [--ceiling]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
CUS, CLOCK_HZ = 256, 2.4e9      # MI355X compute units and peak engine clock
MALL_BYTES = 256 << 20
QWEN_IN, QWEN_OUT = 5120, 17408
SETTLE_S = 0.02   # untimed calls before each workload's timed region (clock settling)
SETTLE_MIN_CALLS = 64
GPU_WARMUP_S = 0.3  # probe launches before the first measurement (a cold GPU ramps its clocks)
LEAD = 16         # untimed calls enqueued between the synchronisation and the start event
REPS = 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_qwen_up_k2.json")
KERNEL_SOURCES = [os.path.join(ROOT, "dequant_gemm_trellis_amd", "csrc", f)
                  for f in ("gemv.hip", "common.hpp")]
HEADLINE_KERNEL = "gemv_kernel<2, false, false, false>"
METRIC = "µs/call and effective HBM GB/s, trellis GEMV 5120→17408 k=2/3/4, M=1"
# probe table kind whose gather rate bounds a kernel's decode: the k = 2 pair
# table, or the eight bank-partitioned codebook copies for k = 3, 4
CEILING_KIND = {2: "pair_b64", 3: "copies8_b32", 4: "copies8_b32"}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the GEMV kernel's sources with comments and whitespace removed,
    so that the stored traffic counters stay valid across comment edits."""
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def n_sets_for(code_bytes: int) -> int:
    return max(2, math.ceil(2 * MALL_BYTES / code_bytes))


class Timer:
    """Event timing of back-to-back calls on torch's current stream."""

    def __init__(self, torch, steps: int, warmup: int):
        self.torch, self.steps, self.warmup = torch, steps, warmup

    def _window(self, launch, i0: int) -> float:
        torch = self.torch
        for i in range(LEAD):
            launch(i0 + i)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(self.steps):
            launch(i0 + LEAD + i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / self.steps

    def run(self, launch) -> dict:
        """launch(i) enqueues call i. Returns ms per call of the first timed
        window and the spread of REPS more."""
        torch = self.torch
        i, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S or i < SETTLE_MIN_CALLS:
            for _ in range(32):
                launch(i)
                i += 1
            torch.cuda.synchronize()
        settle_calls = i
        for _ in range(self.warmup):
            launch(i)
            i += 1
        torch.cuda.synchronize()
        ms = self._window(launch, i)
        i += LEAD + self.steps
        reps = []
        for _ in range(REPS):
            reps.append(self._window(launch, i))
            i += LEAD + self.steps
        reps.sort()
        return {"ms": ms, "reps_us": {"median": reps[REPS // 2] * 1e3, "min": reps[0] * 1e3,
                                      "max": reps[-1] * 1e3},
                "settle_calls": settle_calls}

    def run_graph(self, launch) -> dict:
        """As run, for launch-bound calls: the K calls of a window are captured
        once into a HIP graph (through torch.cuda.graph; the binding enqueues on
        the capturing stream) and each window replays it, so the host's
        per-call cost in the binding does not set the rate."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):   # eager calls before the capture
                launch(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(self.steps):
                launch(i)
        torch.cuda.synchronize()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S or n < 4:
            graph.replay()
            torch.cuda.synchronize()
            n += 1
        for _ in range(self.warmup):
            launch(0)
        torch.cuda.synchronize()

        def window():
            graph.replay()   # lead-in
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record()
            graph.replay()
            end.record()
            torch.cuda.synchronize()
            return start.elapsed_time(end) / self.steps

        ms = window()
        reps = sorted(window() for _ in range(REPS))
        return {"ms": ms, "reps_us": {"median": reps[REPS // 2] * 1e3, "min": reps[0] * 1e3,
                                      "max": reps[-1] * 1e3},
                "settle_calls": n * self.steps, "graph": True}


def summarize(t: dict, code_bytes: int, weights: int, k: int | None, ceiling: dict | None,
              flops: float | None = None) -> dict:
    ms = t["ms"]
    s = ms * 1e-3
    res = {"us_per_call": ms * 1e3, "code_bytes": code_bytes,
           "code_gbps": code_bytes / s / 1e9, "frac_hbm": code_bytes / s / 1e9 / HBM_PEAK_GBS,
           "us_per_call_5_reps": t["reps_us"], "settle_calls": t["settle_calls"]}
    rate = weights / s / CUS / CLOCK_HZ
    res["decode_w_per_clk_cu"] = rate
    if k is not None and ceiling is not None:
        peak = ceiling[CEILING_KIND[k]]["values_per_clk_cu"]
        res["decode_ceiling"] = CEILING_KIND[k]
        res["frac_decode_ceiling"] = rate / peak
    if flops is not None:
        res["mfma_frac"] = flops / s / 1e12 / MFMA_BF16_PEAK_TFLOPS
    return res


class Pool:
    """Rotating device-resident code sets of the 17408 x 5120 stored matrix
    at bit width k, each with its own codebook and row scales."""

    def __init__(self, T, torch, dev, k: int):
        import numpy as np

        from dequant_gemm_trellis_amd import synth

        self.k = k
        self.shape = synth.Shape(1, 256, 12, k, QWEN_IN, QWEN_OUT)
        self.code_bytes = self.shape.rows * self.shape.words_per_row * 4
        self.n = n_sets_for(self.code_bytes)
        cfg = synth.CONFIG_IDS["qwen_up_gemv"]
        self.items = []
        for i in range(self.n):
            codes = synth.codes(self.shape, cfg, proj=i)
            self.items.append((torch.from_numpy(codes.view(np.int32)).to(dev),
                               torch.from_numpy(synth.scales(self.shape, cfg, proj=i)).to(dev),
                               T.lut_upload(synth.lut(self.shape, cfg, proj=i), device=dev)))
            if i == 0:
                self.first = synth.make_problem(self.shape, 1, cfg, proj=0)

    def set(self, i):
        return self.items[i % self.n]


def device_x(torch, dev, shape, M, cfg, proj=0):
    import numpy as np

    from dequant_gemm_trellis_amd import synth

    x = synth.activations(shape, cfg, M, proj)
    t = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return t.reshape(-1) if M == 1 else t


# ----------------------------------------------------------------------------- ceiling
def measure_ceiling(T, torch, dev) -> dict:
    """Random LDS gather rate of the three decode-table layouts, in decoded
    weights per clock per CU at the nominal 2.4 GHz (the unit of every decode
    figure here): the difference of two launches of the probe kernel."""
    out = torch.empty(T.gather_probe_out_floats(), dtype=torch.float32, device=dev)
    r1, r2 = 64, 320
    t0 = time.perf_counter()   # the first measurement of the run: warm the GPU up first
    while time.perf_counter() - t0 < GPU_WARMUP_S:
        for _ in range(8):
            T.gather_probe(T.PROBE_PAIR_B64, r2, out)
        torch.cuda.synchronize()
    res = {}
    for kind, name in ((T.PROBE_PAIR_B64, "pair_b64"), (T.PROBE_COPIES8_B32, "copies8_b32"),
                       (T.PROBE_SINGLE_B32, "single_b32")):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(4):
                T.gather_probe(kind, r2, out)
            torch.cuda.synchronize()
        deltas = []
        for _ in range(REPS):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            T.gather_probe(kind, r1, out)          # lead-in
            ev[0].record()
            v1 = T.gather_probe(kind, r1, out)
            ev[1].record()
            ev[2].record()
            v2 = T.gather_probe(kind, r2, out)
            ev[3].record()
            torch.cuda.synchronize()
            dt = (ev[2].elapsed_time(ev[3]) - ev[0].elapsed_time(ev[1])) * 1e-3
            deltas.append((v2 - v1) / dt)
        deltas.sort()
        per_s = deltas[REPS // 2]
        vpr = 2 if name == "pair_b64" else 1
        rate = per_s / CUS / CLOCK_HZ
        res[name] = {"values_per_clk_cu": rate,
                     "clk_per_wave_read": 64 * vpr / rate,
                     "values_per_s": per_s}
    return res


# ----------------------------------------------------------------------------- workloads
def bench_all(T, torch, dev, timer: Timer, ceiling: dict | None, only=None, extra=False) -> dict:
    from dequant_gemm_trellis_amd import synth

    C = synth.CONFIG_IDS
    W = QWEN_IN * QWEN_OUT   # weights per projection
    out = {}

    def want(name):
        return only is None or name in only

    def record(name, launch, code_bytes, weights, k, flops=None, graph=False, **info):
        log(f"bench: {name}")
        t = timer.run_graph(launch) if graph else timer.run(launch)
        out[name] = {**summarize(t, code_bytes, weights, k, ceiling, flops), **info}
        log(f"bench: {name}: {out[name]['us_per_call']:.2f} us/call, "
            f"{out[name]['code_gbps']:.0f} GB/s")

    # C1: tiny GEMV, one resident set (launch-bound)
    if want("c1_tiny_gemv_k2"):
        sh = synth.Shape(1, 256, 12, 2, 512, 256)
        p = synth.make_problem(sh, 1, C["tiny_gemv"])
        import numpy as np

        codes = torch.from_numpy(p.codes.view(np.int32)).to(dev)
        scales = torch.from_numpy(p.scales).to(dev)
        lut = T.lut_upload(p.lut, device=dev)
        x = torch.from_numpy(p.x.view(np.int16)).to(dev).view(torch.bfloat16).reshape(-1)
        y = torch.empty(256, dtype=torch.bfloat16, device=dev)
        g = T.Geometry.of(sh)
        record("c1_tiny_gemv_k2", lambda i: T.gemv(x, codes, scales, lut, g, y=y),
               codes.numel() * 4, 512 * 256, None, graph=True, rotation_sets=1, bound="launch",
               note="launch-bound: the timed calls replay a captured HIP graph")

    pools = {}

    def pool(k):
        if k not in pools:
            log(f"bench: generating rotating code sets, k={k}")
            pools[k] = Pool(T, torch, dev, k)
        return pools[k]

    first = None
    # C2: the GEMV at k = 2, 3, 4 (k = 2 is the headline)
    for k in (2, 3, 4):
        name = f"c2_gemv_k{k}"
        if not want(name):
            continue
        pl = pool(k)
        x = device_x(torch, dev, pl.shape, 1, C["qwen_up_gemv"])
        y = torch.empty(QWEN_OUT, dtype=torch.bfloat16, device=dev)
        g = T.Geometry.of(pl.shape)
        record(name, lambda i: T.gemv(x, *pl.set(i), g, y=y), pl.code_bytes, W, k,
               rotation_sets=pl.n)
        if k == 2:
            first = pl.first
            # all-operand algorithmic bytes: codes, scales, x, y, codebook
            alg = pl.code_bytes + 4 * QWEN_OUT + 2 * QWEN_IN + 2 * QWEN_OUT + 4 * 4096
            out[name]["alg_bytes"] = alg
            out[name]["alg_gbps"] = alg / (out[name]["us_per_call"] * 1e-6) / 1e9

    # C3: the axis-0 scatter at k = 3 (the same code sets read as 17408 x 5120, axis 0)
    if want("c3_scatter_k3"):
        pl = pool(3)
        sh0 = synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN)
        g0 = T.Geometry.of(sh0)
        x = device_x(torch, dev, sh0, 1, C["qwen_down_scatter"])
        y = torch.empty(QWEN_IN, dtype=torch.bfloat16, device=dev)
        nbytes = T.workspace_bytes(g0, 1, T.OP_GEMV_SCATTER)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        record("c3_scatter_k3", lambda i: T.gemv_scatter(x, *pl.set(i), g0, workspace=ws, y=y),
               pl.code_bytes, W, 3, rotation_sets=pl.n, workspace_bytes=nbytes)

    # C4: prefill, k = 2, 3, 4 x M = 5, 8, 16, 32
    for k in (2, 3, 4):
        for M in (5, 8, 16, 32):
            name = f"c4_prefill_k{k}_M{M}"
            if not want(name):
                continue
            pl = pool(k)
            x = device_x(torch, dev, pl.shape, M, C["qwen_up_prefill"])
            y = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
            g = T.Geometry.of(pl.shape)
            nws = T.workspace_bytes(g, M, T.OP_PREFILL)
            ws = torch.empty(nws // 4, dtype=torch.float32, device=dev) if nws else None
            record(name, lambda i, ws=ws: T.prefill(x, *pl.set(i), g, workspace=ws, y=y),
                   pl.code_bytes, W, k, flops=2.0 * M * W, rotation_sets=pl.n)

    # C5: MLP, gate + up in one launch, then down (axis 0), k = 4, M = 1 and 32
    for M in (1, 32):
        name = f"c5_mlp_k4_M{M}"
        if not want(name):
            continue
        pl = pool(4)
        sh1 = pl.shape
        sh0 = synth.Shape(0, 256, 12, 4, QWEN_OUT, QWEN_IN)
        g1, g0 = T.Geometry.of(sh1), T.Geometry.of(sh0)
        x = device_x(torch, dev, sh1, M, C["qwen_mlp"])
        xd = device_x(torch, dev, sh0, M, C["qwen_mlp"], proj=2)
        ya = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
        yb = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((M, QWEN_IN), dtype=torch.bfloat16, device=dev)
        op = T.OP_GEMV_SCATTER if M == 1 else T.OP_PREFILL
        ws = torch.empty(T.workspace_bytes(g0, M, op) // 4, dtype=torch.float32, device=dev)

        def mlp(i, M=M, x=x, xd=xd, ya=ya, yb=yb, yd=yd, ws=ws, g1=g1, g0=g0):
            a, b, d = pl.set(3 * i), pl.set(3 * i + 1), pl.set(3 * i + 2)
            if M == 1:
                T.gemv_dual(x, a, b, g1, y_a=ya.reshape(-1), y_b=yb.reshape(-1))
                T.gemv_scatter(xd, *d, g0, workspace=ws, y=yd.reshape(-1))
            else:
                T.prefill_dual(x, a, b, g1, y_a=ya, y_b=yb)
                T.prefill(xd, *d, g0, workspace=ws, y=yd)

        record(name, mlp, 3 * pl.code_bytes, 3 * W, 4, flops=2.0 * M * 3 * W, rotation_sets=pl.n,
               note="gate and up read the same activations in one launch; down reads its own")

    # C5 as a chained layer: gate + up with the fused SwiGLU epilogue, whose
    # output h feeds the down projection
    for M in (1, 32):
        name = f"c5_mlp_swiglu_k4_M{M}"
        if not want(name):
            continue
        pl = pool(4)
        sh1 = pl.shape
        sh0 = synth.Shape(0, 256, 12, 4, QWEN_OUT, QWEN_IN)
        g1, g0 = T.Geometry.of(sh1), T.Geometry.of(sh0)
        x = device_x(torch, dev, sh1, M, C["qwen_mlp"])
        h = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((M, QWEN_IN), dtype=torch.bfloat16, device=dev)
        op = T.OP_GEMV_SCATTER if M == 1 else T.OP_PREFILL
        ws = torch.empty(T.workspace_bytes(g0, M, op) // 4, dtype=torch.float32, device=dev)
        x2 = x.reshape(M, -1)

        def mlp_sw(i, M=M, x2=x2, h=h, yd=yd, ws=ws, g1=g1, g0=g0):
            a, b, d = pl.set(3 * i), pl.set(3 * i + 1), pl.set(3 * i + 2)
            T.gate_up_swiglu(x2, a, b, g1, h=h)
            if M == 1:
                T.gemv_scatter(h.reshape(-1), *d, g0, workspace=ws, y=yd.reshape(-1))
            else:
                T.prefill(h, *d, g0, workspace=ws, y=yd)

        record(name, mlp_sw, 3 * pl.code_bytes, 3 * W, 4, flops=2.0 * M * 3 * W,
               rotation_sets=pl.n,
               note="gate and up with the fused SwiGLU epilogue (one launch), its output "
                    "feeding down: a whole MLP layer")

    if extra:
        extra_workloads(T, torch, dev, timer, ceiling, pool, out, only)
    for k in list(pools):
        del pools[k]
    torch.cuda.empty_cache()
    return out, first


def extra_workloads(T, torch, dev, timer, ceiling, pool, out, only):
    """Workloads beyond the five configurations: block-interleaved codes, the
    small-batch row counts M = 2 / 4, axis 0 at M = 2 / 4 / 8, and the MLP with
    separate gate and up launches."""
    from dequant_gemm_trellis_amd import synth

    C = synth.CONFIG_IDS
    W = QWEN_IN * QWEN_OUT

    def want(name):
        return only is None or name in only

    def record(name, launch, code_bytes, weights, k, flops=None, **info):
        log(f"bench: {name}")
        out[name] = {**summarize(timer.run(launch), code_bytes, weights, k, ceiling, flops), **info}

    if want("x_gemv_k2_interleave2"):
        pl = pool(2)
        sh = synth.Shape(1, 256, 12, 2, QWEN_IN, QWEN_OUT, 2)
        g = T.Geometry.of(sh)
        x = device_x(torch, dev, sh, 1, C["qwen_up_gemv"])
        y = torch.empty(QWEN_OUT, dtype=torch.bfloat16, device=dev)
        record("x_gemv_k2_interleave2", lambda i: T.gemv(x, *pl.set(i), g, y=y), pl.code_bytes,
               W, 2, note="the same uniform random words read in the block-pair layout")
    if want("x_scatter_k3_interleave2"):
        pl = pool(3)
        sh0 = synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN, 2)
        g0 = T.Geometry.of(sh0)
        x = device_x(torch, dev, sh0, 1, C["qwen_down_scatter"])
        y = torch.empty(QWEN_IN, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(T.workspace_bytes(g0, 1, T.OP_GEMV_SCATTER) // 4, dtype=torch.float32,
                         device=dev)
        record("x_scatter_k3_interleave2",
               lambda i: T.gemv_scatter(x, *pl.set(i), g0, workspace=ws, y=y), pl.code_bytes, W, 3)
    for k in (2, 3, 4):
        for M in (2, 4):
            name = f"x_prefill_k{k}_M{M}"
            if not want(name):
                continue
            pl = pool(k)
            x = device_x(torch, dev, pl.shape, M, C["qwen_up_prefill"])
            y = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
            g = T.Geometry.of(pl.shape)
            record(name, lambda i: T.prefill(x, *pl.set(i), g, y=y), pl.code_bytes, W, k,
                   flops=2.0 * M * W)
    for M in (2, 4, 8, 32):
        name = f"x_prefill_axis0_k3_M{M}"
        if not want(name):
            continue
        pl = pool(3)
        sh0 = synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN)
        g0 = T.Geometry.of(sh0)
        x = device_x(torch, dev, sh0, M, C["qwen_down_scatter"])
        y = torch.empty((M, QWEN_IN), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(T.workspace_bytes(g0, M, T.OP_PREFILL) // 4, dtype=torch.float32,
                         device=dev)
        record(name, lambda i: T.prefill(x, *pl.set(i), g0, workspace=ws, y=y), pl.code_bytes,
               W, 3, flops=2.0 * M * W)
    for M in (1, 8, 32):
        name = f"x_mlp_k4_M{M}_separate"
        if not want(name):
            continue
        pl = pool(4)
        sh1 = pl.shape
        sh0 = synth.Shape(0, 256, 12, 4, QWEN_OUT, QWEN_IN)
        g1, g0 = T.Geometry.of(sh1), T.Geometry.of(sh0)
        x = device_x(torch, dev, sh1, M, C["qwen_mlp"])
        xd = device_x(torch, dev, sh0, M, C["qwen_mlp"], proj=2)
        ys = [torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        yd = torch.empty((M, QWEN_IN), dtype=torch.bfloat16, device=dev)
        op = T.OP_GEMV_SCATTER if M == 1 else T.OP_PREFILL
        ws = torch.empty(T.workspace_bytes(g0, M, op) // 4, dtype=torch.float32, device=dev)

        def mlp_sep(i, M=M, x=x, xd=xd, ys=ys, yd=yd, ws=ws, g1=g1, g0=g0):
            for j in range(2):
                s = pl.set(3 * i + j)
                if M == 1:
                    T.gemv(x, *s, g1, y=ys[j].reshape(-1))
                else:
                    T.prefill(x, *s, g1, y=ys[j])
            d = pl.set(3 * i + 2)
            if M == 1:
                T.gemv_scatter(xd, *d, g0, workspace=ws, y=yd.reshape(-1))
            else:
                T.prefill(xd, *d, g0, workspace=ws, y=yd)

        record(name, mlp_sep, 3 * pl.code_bytes, 3 * W, 4, flops=2.0 * M * 3 * W)


# ----------------------------------------------------------------------------- oracle baseline
def cpu_baseline(p, seconds: float):
    """The oracle (single-threaded C, float64 accumulation) on whole output rows
    of the same k = 2 GEMV, repeated in 2176-row chunks until `seconds` pass;
    scaled to a full call."""
    import oracle

    s = p.shape
    chunk = 2176
    rows_done, t0 = 0, time.perf_counter()
    while True:
        r0 = rows_done % s.rows
        r1 = min(s.rows, r0 + chunk)
        oracle.fused_f64(p.x, p.codes[r0:r1], p.scales[r0:r1], p.lut, 1, s.T, s.L, s.k,
                         s.in_features, r1 - r0)
        rows_done += r1 - r0
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_call = el * s.rows / rows_done
    code_bytes = s.rows * s.words_per_row * 4
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": code_bytes / per_call / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_call": per_call * 1e6, "host_cpu": cpu_model,
            "sample": f"{rows_done} output rows x 5120 inputs of the k=2 GEMV "
                      f"({el:.1f} s), scaled to the full 17408-row call; "
                      f"host has {os.cpu_count()} logical cores"}


def traffic_entry():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the current kernel source; else None."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--extra", action="store_true",
                    help="also time interleaved codes, M = 2/4, axis 0 at M = 2..32, separate MLP")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", default="",
                    help="comma-separated workload names to time (profiling runs)")
    ap.add_argument("--ceiling", action="store_true",
                    help="measure only the LDS gather ceiling and print it")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain device copy of 512 MiB (scales the FETCH_SIZE/WRITE_SIZE "
                         "counters of the traffic figure) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the kernels run on one GPU (a GPU's share of a sharded layer is the "
              "same kernel on fewer rows); nothing here runs across GPUs, so --gpus must be 1.",
              file=sys.stderr)
        return 2

    import torch

    if not os.path.exists(os.path.join(ROOT, "dequant_gemm_trellis_amd", "libtrellis.so")):
        import __graft_entry__

        __graft_entry__.build()
    from dequant_gemm_trellis_amd import trellis as T

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        n = 512 << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return 0

    log("bench: decode ceiling (LDS gather probe)")
    ceiling = measure_ceiling(T, torch, dev)
    log(f"bench: ceiling {json.dumps(ceiling)}")
    if args.ceiling:
        print(json.dumps({"decode_ceiling": ceiling, "unit": "decoded weights/clk/CU at 2.4 GHz",
                          "cus": CUS}), flush=True)
        return 0

    only = set(args.only.split(",")) if args.only else None
    timer = Timer(torch, args.steps, args.warmup)
    work, first = bench_all(T, torch, dev, timer, ceiling, only, args.extra)

    cpu = None
    if not args.no_cpu and first is not None:
        log("bench: oracle cpu baseline")
        cpu = cpu_baseline(first, args.cpu_seconds)

    head = work.get("c2_gemv_k2") or next(iter(work.values()))
    achieved = head["code_gbps"]
    line = {
        "metric": METRIC,
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_call"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded uniform u32 codes, N(0,1) f32 codebook, U[0.5,1.5) f32 "
                "scales, N(0,1) bf16 x)",
        "config": {"workload": "trellis GEMV qwen-mlp up-projection, axis 1, in 5120 -> out "
                               "17408, T 256, L 12, k 2, M 1 (all five configurations in "
                               "workloads)",
                   "k": 2, "M": 1, "in_features": QWEN_IN, "out_features": QWEN_OUT,
                   "rotation_sets": head.get("rotation_sets")},
        "timing": {"settle_s": SETTLE_S, "settle_min_calls": SETTLE_MIN_CALLS,
                   "gpu_warmup_s": GPU_WARMUP_S, "lead_in_calls": LEAD, "reps": REPS,
                   "clock_hz_nominal": CLOCK_HZ, "cus": CUS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_entry(), "kernel": HEADLINE_KERNEL,
                     "bytes_per_launch": head["code_bytes"]},
        "decode": {"bound": "lds_gather", "unit": "weights/clk/CU",
                   "achieved": round(head["decode_w_per_clk_cu"], 3),
                   "peak": round(ceiling["pair_b64"]["values_per_clk_cu"], 3),
                   "frac": round(head.get("frac_decode_ceiling", 0.0), 4),
                   "peak_source": "trellis_gather_probe, pair_b64, measured in this run"},
        "decode_ceiling": ceiling,
        "workloads": work,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
