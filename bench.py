#!/usr/bin/env python3
"""Benchmark of the trellis dequantize-and-multiply hot path on one MI355X.

Workload (the headline): the axis-1 trellis GEMV of the Qwen MLP up
projection, in 5120 -> out 17408, T 256, L 12, M 1, bf16 activations, f32
scales, a 4096-entry f32 codebook, seeded uniform random u32 codes. One step
is one GEMV call (codebook staging, code streaming, window decode, codebook
gather, scale + bf16 rounding, MFMA dot, reduction, bf16 store). The value is
the effective HBM bandwidth on packed-code bytes for k = 2; k = 3 and k = 4 are
timed the same way and reported beside it.

Inputs are resident in HBM before timing starts. Calls rotate over enough
distinct input sets (>= 2 x 256 MB of codes) that the 256 MB Infinity Cache
cannot hold them, so the figure is HBM-bound, not cache-bound.

Timing: HIP events recorded on the stream the kernels are launched on (torch's
current stream, which the binding passes to the C ABI), around exactly K
back-to-back calls after W warm-up calls, bracketed by device synchronisation.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra] [--no-cpu]
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
# Codebook-gather ceiling, decoded weights per clock per CU, measured on MI355X
# with a random-index LDS gather microbenchmark (uniform random indices into a
# 128 KB table, 512-thread workgroups, 8 waves per CU): ds_read_b64 as from the
# k = 2 pair table (two weights per lane, 7.21 clocks per wave-wide read) and
# ds_read_b32 from eight bank-partitioned codebook copies as the k = 3, 4 GEMV
# reads them (6.14 clocks; a single copy gives 8.4 values per clock).
GATHER_PEAK_W_PER_CLK = {2: 17.75, 3: 10.43, 4: 10.43}
MALL_BYTES = 256 << 20
QWEN_IN, QWEN_OUT = 5120, 17408
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_qwen_up_k2.json")
KERNEL_SOURCES = [os.path.join(ROOT, "dequant_gemm_trellis_amd", "csrc", f)
                  for f in ("gemv.hip", "common.hpp")]
METRIC = "µs/call and effective HBM GB/s, trellis GEMV 5120→17408 k=2/3/4, M=1"


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


class Sets:
    """Rotating device-resident input sets for one projection shape."""

    def __init__(self, shape, M, cfg, n_sets, T, torch, dev, proj0=0):
        import numpy as np

        from dequant_gemm_trellis_amd import synth

        self.shape, self.M = shape, M
        self.items = []
        for i in range(n_sets):
            p = synth.make_problem(shape, M, cfg, proj=proj0 + i)
            codes = torch.from_numpy(p.codes.view(np.int32)).to(dev)
            scales = torch.from_numpy(p.scales).to(dev)
            x = torch.from_numpy(p.x.view(np.int16)).to(dev).view(torch.bfloat16)
            if M == 1:
                x = x.reshape(-1)
            lut = T.lut_upload(p.lut, device=dev)
            self.items.append((x, codes, scales, lut))
            if i == 0:
                self.first = p
        self.code_bytes = self.items[0][1].numel() * 4


def n_sets_for(code_bytes: int) -> int:
    return max(2, math.ceil(2 * MALL_BYTES / code_bytes))


def time_calls(torch, launch, n_items, steps, warmup):
    """ms per call over exactly `steps` back-to-back calls (events on the
    current stream, synchronised on both sides)."""
    for i in range(warmup):
        launch(i % n_items)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        launch(i % n_items)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def gemv_bench(T, torch, dev, k, steps, warmup):
    from dequant_gemm_trellis_amd import synth

    shape = synth.Shape(1, 256, 12, k, QWEN_IN, QWEN_OUT)
    code_bytes = shape.rows * shape.words_per_row * 4
    sets = Sets(shape, 1, synth.CONFIG_IDS["qwen_up_gemv"], n_sets_for(code_bytes), T, torch, dev)
    y = torch.empty(QWEN_OUT, dtype=torch.bfloat16, device=dev)
    geom = T.Geometry.of(shape)

    def launch(i):
        x, codes, scales, lut = sets.items[i]
        T.gemv(x, codes, scales, lut, geom, y=y)

    ms = time_calls(torch, launch, len(sets.items), steps, warmup)
    # five more timed runs of the same length: the spread behind the one figure
    reps = sorted(time_calls(torch, launch, len(sets.items), steps, 0) * 1e3 for _ in range(5))
    warm = time_calls(torch, lambda i: launch(0), 1, max(steps // 4, 10), 5)
    # every byte the call must move: codes, scales, x, y and the codebook
    alg_bytes = code_bytes + 4 * shape.rows + 2 * shape.cols + 2 * shape.rows + 4 * 4096
    res = {"us_per_call": ms * 1e3, "gbps": code_bytes / (ms * 1e-3) / 1e9,
           "alg_bytes": alg_bytes, "alg_gbps": alg_bytes / (ms * 1e-3) / 1e9,
           "frac_hbm": code_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "decode_w_per_clk_cu": shape.rows * shape.cols / (ms * 1e-3) / CUS / CLOCK_HZ,
           "frac_decode_ceiling": shape.rows * shape.cols / (ms * 1e-3) / CUS / CLOCK_HZ
                                  / GATHER_PEAK_W_PER_CLK[k],
           "us_per_call_5_reps": {"median": reps[2], "min": reps[0], "max": reps[4]},
           "code_bytes": code_bytes, "rotation_sets": len(sets.items),
           "us_per_call_mall_resident": warm * 1e3}
    first = sets.first
    del sets
    torch.cuda.empty_cache()
    return res, first


def extra_bench(T, torch, dev, steps, warmup, only=None):
    """Other workloads: axis-0 scatter k=3 (and its geometry at M=2/4/8), prefill
    M=2/4/5/8/16/32, MLP k=4 M=1/8/32,
    and the scatter and the k=2 GEMV on block-interleave-2 codes (the same
    uniform random words, read in the pair layout)."""
    from dequant_gemm_trellis_amd import synth

    out = {}
    C = synth.CONFIG_IDS

    def want(*names):
        return only is None or any(n in only for n in names)

    if want("scatter_qwen_down_k3", "scatter_qwen_down_k3_interleave2"):
        scatter_bench(T, torch, dev, steps, warmup, only, out)
    if want("gemv_qwen_up_k2_interleave2"):
        sh = synth.Shape(1, 256, 12, 2, QWEN_IN, QWEN_OUT, 2)
        cb = sh.rows * sh.words_per_row * 4
        sets = Sets(sh, 1, C["qwen_up_gemv"], n_sets_for(cb), T, torch, dev)
        y = torch.empty(QWEN_OUT, dtype=torch.bfloat16, device=dev)
        g2 = T.Geometry.of(sh)
        ms = time_calls(torch, lambda i: T.gemv(*sets.items[i], g2, y=y), len(sets.items), steps,
                        warmup)
        out["gemv_qwen_up_k2_interleave2"] = {"us_per_call": ms * 1e3,
                                              "gbps": cb / (ms * 1e-3) / 1e9}
        del sets
    for k in (2, 3, 4):
        sh = synth.Shape(1, 256, 12, k, QWEN_IN, QWEN_OUT)
        cb = sh.rows * sh.words_per_row * 4
        for M in (2, 4, 5, 8, 16, 32):
            name = f"prefill_qwen_up_k{k}_M{M}"
            if not want(name):
                continue
            sets = Sets(sh, M, C["qwen_up_prefill"], n_sets_for(cb), T, torch, dev)
            y = torch.empty((M, QWEN_OUT), dtype=torch.bfloat16, device=dev)
            g = T.Geometry.of(sh)
            ms = time_calls(torch, lambda i: T.prefill(*sets.items[i], g, y=y),
                            len(sets.items), steps, warmup)
            flops = 2.0 * M * QWEN_IN * QWEN_OUT
            out[name] = {"us_per_call": ms * 1e3, "gbps": cb / (ms * 1e-3) / 1e9,
                         "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
            del sets
    # axis 0 at the scatter's geometry with several activation rows (decode once per row set)
    sh = synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN)
    cb = sh.rows * sh.words_per_row * 4
    for M in (2, 4, 8):
        name = f"prefill_qwen_down_k3_M{M}"
        if not want(name):
            continue
        sets = Sets(sh, M, C["qwen_down_scatter"], n_sets_for(cb), T, torch, dev)
        y = torch.empty((M, QWEN_IN), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(T.workspace_bytes(sh, M, T.OP_PREFILL) // 4, dtype=torch.float32,
                         device=dev)
        g = T.Geometry.of(sh)
        ms = time_calls(torch, lambda i: T.prefill(*sets.items[i], g, workspace=ws, y=y),
                        len(sets.items), steps, warmup)
        out[name] = {"us_per_call": ms * 1e3, "gbps": cb / (ms * 1e-3) / 1e9}
        del sets
    for M in (1, 8, 32):
        if want(f"mlp_k4_M{M}"):
            mlp_bench(T, torch, dev, M, steps, warmup, out)
    torch.cuda.empty_cache()
    return out


def scatter_bench(T, torch, dev, steps, warmup, only, out):
    """Axis-0 scatter k=3, on row-major and on block-interleave-2 codes."""
    from dequant_gemm_trellis_amd import synth

    C = synth.CONFIG_IDS
    sh = synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN)
    cb = sh.rows * sh.words_per_row * 4
    sets = Sets(sh, 1, C["qwen_down_scatter"], n_sets_for(cb), T, torch, dev)
    ws = torch.empty(T.workspace_bytes(sh, 1, T.OP_GEMV_SCATTER) // 4, dtype=torch.float32,
                     device=dev)
    y = torch.empty(QWEN_IN, dtype=torch.bfloat16, device=dev)
    g = T.Geometry.of(sh)
    ms = time_calls(torch, lambda i: T.gemv_scatter(*sets.items[i], g, workspace=ws, y=y),
                    len(sets.items), steps, warmup)
    out["scatter_qwen_down_k3"] = {"us_per_call": ms * 1e3, "gbps": cb / (ms * 1e-3) / 1e9}
    g2 = T.Geometry.of(synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN, 2))
    ms = time_calls(torch, lambda i: T.gemv_scatter(*sets.items[i], g2, workspace=ws, y=y),
                    len(sets.items), steps, warmup)
    out["scatter_qwen_down_k3_interleave2"] = {"us_per_call": ms * 1e3,
                                               "gbps": cb / (ms * 1e-3) / 1e9}
    del sets


def mlp_bench(T, torch, dev, M, steps, warmup, out):
    """The MLP workload: gate and up (axis 1, the same activations, in one
    launch through the dual entry points, also timed as two separate calls)
    then down (axis 0), k=4."""
    from dequant_gemm_trellis_amd import synth

    C = synth.CONFIG_IDS
    shapes = [synth.Shape(1, 256, 12, 4, QWEN_IN, QWEN_OUT),
              synth.Shape(1, 256, 12, 4, QWEN_IN, QWEN_OUT),
              synth.Shape(0, 256, 12, 4, QWEN_OUT, QWEN_IN)]
    cb = 3 * shapes[0].rows * shapes[0].words_per_row * 4
    n = n_sets_for(cb)
    projs = [Sets(s, M, C["qwen_mlp"], n, T, torch, dev, proj0=10 * j)
             for j, s in enumerate(shapes)]
    geoms = [T.Geometry.of(s) for s in shapes]
    ys = [torch.empty((M, s.out_features), dtype=torch.bfloat16, device=dev) for s in shapes]
    ws = torch.empty(max(T.workspace_bytes(shapes[2], M, T.OP_PREFILL), 16) // 4,
                     dtype=torch.float32, device=dev)

    ws1 = ws[: T.workspace_bytes(shapes[2], 1, T.OP_GEMV_SCATTER) // 4]

    def down(i):
        x, codes, scales, lut = projs[2].items[i]
        if M == 1:
            T.gemv_scatter(x, codes, scales, lut, geoms[2], workspace=ws1, y=ys[2].reshape(-1))
        else:
            T.prefill(x, codes, scales, lut, geoms[2], workspace=ws, y=ys[2])

    def mlp(i):
        # gate and up read the same activations (the gate set's x)
        x = projs[0].items[i][0]
        if M == 1:
            T.gemv_dual(x, projs[0].items[i][1:], projs[1].items[i][1:], geoms[0],
                        y_a=ys[0].reshape(-1), y_b=ys[1].reshape(-1))
        else:
            T.prefill_dual(x, projs[0].items[i][1:], projs[1].items[i][1:], geoms[0],
                           y_a=ys[0], y_b=ys[1])
        down(i)

    def mlp_separate(i):
        x = projs[0].items[i][0]
        for j in range(2):
            _, codes, scales, lut = projs[j].items[i]
            if M == 1:
                T.gemv(x, codes, scales, lut, geoms[j], y=ys[j].reshape(-1))
            else:
                T.prefill(x, codes, scales, lut, geoms[j], y=ys[j])
        down(i)

    ms = time_calls(torch, mlp, n, max(steps // 3, 10), warmup)
    out[f"mlp_k4_M{M}"] = {"us_per_call": ms * 1e3, "gbps": cb / (ms * 1e-3) / 1e9}
    ms = time_calls(torch, mlp_separate, n, max(steps // 3, 10), warmup)
    name = "mlp_k4_M1_separate_gemvs" if M == 1 else f"mlp_k4_M{M}_separate_prefills"
    out[name] = {"us_per_call": ms * 1e3, "gbps": cb / (ms * 1e-3) / 1e9}
    del projs


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
    ap.add_argument("--steps", type=int, default=2000)
    # about 15 ms of GEMV calls: shorter warm-ups (50 calls) timed 3-5% slower
    # than the same calls repeated right afterwards
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--extra", action="store_true", help="also time scatter, prefill and MLP")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only-k", type=int, default=0, help="time only this k (profiling runs)")
    ap.add_argument("--only-extra", default="",
                    help="comma-separated extra workload names to time (implies --extra; "
                         "profiling runs)")
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

    per_k, first = {}, None
    for k in ((args.only_k,) if args.only_k else (2, 3, 4)):
        log(f"bench: gemv k={k} steps={args.steps} warmup={args.warmup}")
        per_k[str(k)], p = gemv_bench(T, torch, dev, k, args.steps, args.warmup)
        if k == 2:
            first = p
        log(f"bench: gemv k={k}: {json.dumps(per_k[str(k)])}")
    head = per_k.get("2") or next(iter(per_k.values()))

    extra = None
    if args.extra or args.only_extra:
        log("bench: extra workloads")
        extra = extra_bench(T, torch, dev, max(args.steps // 4, 20), max(args.warmup // 4, 10),
                            only=set(args.only_extra.split(",")) if args.only_extra else None)

    cpu = None
    if not args.no_cpu and first is not None:
        log("bench: oracle cpu baseline")
        cpu = cpu_baseline(first, args.cpu_seconds)

    achieved = head["gbps"]
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
                               "17408, T 256, L 12, k 2 (k 3/4 in per_k), M 1",
                   "k": 2, "M": 1, "in_features": QWEN_IN, "out_features": QWEN_OUT,
                   "rotation_sets": head["rotation_sets"]},
        "per_k": per_k,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_entry(),
                     "kernel": "gemv_kernel<2, false>",
                     "bytes_per_launch": head["code_bytes"]},
        "decode": {"bound": "lds_gather", "unit": "weights/clk/CU",
                   "achieved": round(head["decode_w_per_clk_cu"], 3),
                   "peak": GATHER_PEAK_W_PER_CLK[2],
                   "frac": round(head["frac_decode_ceiling"], 4)},
        "cpu_baseline": cpu,
    }
    if extra is not None:
        line["extra"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
