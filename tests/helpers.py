"""Shared helpers for the GPU parity tests: device upload of seeded problems,
the output tolerance gate, and bf16 conversions. No decoding arithmetic."""
from __future__ import annotations

import sys

import numpy as np

from dequant_gemm_trellis_amd import synth

QWEN_IN, QWEN_OUT = 5120, 17408
TOL = 1e-2  # max relative error on bf16 outputs (float32 accumulation)


def say(msg: str) -> None:
    """Name the case before a GPU step, so a failed box still tells which one."""
    print(msg, flush=True)
    sys.stdout.flush()


def gate(y: np.ndarray, ref: np.ndarray) -> float:
    """max_i |y_i - ref_i| / max(|ref_i|, 1e-3 * max_j |ref_j|): a relative error
    floored near zero so a well-conditioned bf16 result is not failed by a
    cancellation-sized reference value."""
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    floor = 1e-3 * np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), floor)))


class Dev:
    """A seeded problem resident on the GPU."""

    def __init__(self, p: synth.Problem, T, device="cuda"):
        import torch

        self.p = p
        self.shape = p.shape
        self.codes = torch.from_numpy(p.codes.view(np.int32)).to(device)
        self.scales = torch.from_numpy(p.scales).to(device)
        self.x = torch.from_numpy(p.x.view(np.int16)).to(device).view(torch.bfloat16)
        self.lut = T.lut_upload(p.lut, device=device)


def bf16_to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_bits(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def with_x(p: synth.Problem, x_bits: np.ndarray) -> synth.Problem:
    return synth.Problem(p.shape, x_bits.shape[0], p.codes, p.lut, p.scales, x_bits)


def row_subset(p: synth.Problem, rows: np.ndarray) -> synth.Problem:
    """The same codes restricted to some stored rows (shape shrinks along rows)."""
    s = p.shape
    n = len(rows)
    if s.axis == 1:
        shape = synth.Shape(1, s.T, s.L, s.k, s.in_features, n)
        x = p.x
    else:
        shape = synth.Shape(0, s.T, s.L, s.k, n, s.out_features)
        x = np.ascontiguousarray(p.x[:, rows])
    return synth.Problem(shape, p.M, np.ascontiguousarray(p.codes[rows]), p.lut,
                         np.ascontiguousarray(p.scales[rows]), x)



def oracle_columns(fn, n_out: int, workers: int = 16, chunk: int = 256):
    """Run fn(n_begin, n_end) -> array [M, n_out] (zeros outside the range) over
    column chunks on a thread pool and add the results: the oracle's C code
    releases the GIL, so a full-size reference takes seconds instead of
    minutes. Each column is still computed by the oracle alone."""
    import concurrent.futures as cf

    bounds = [(b, min(n_out, b + chunk)) for b in range(0, n_out, chunk)]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(lambda be: (be, fn(*be)), bounds))
    out = None
    for (b, e), a in parts:
        if out is None:
            out = np.zeros_like(a)
        out[:, b:e] = a[:, b:e]
    return out


def oracle_y_full(p: synth.Problem, workers: int = 16):
    """The oracle's whole output for a problem ([M, out] float64), columns
    computed in parallel chunks (oracle_columns)."""
    import oracle

    s = p.shape
    return oracle_columns(
        lambda b, e: oracle.fused_f64(p.x, p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k,
                                      s.in_features, s.out_features, b, e,
                                      block_interleave=s.block_interleave),
        s.out_features, workers)


def oracle_W_full(p: synth.Problem, workers: int = 16, chunk: int = 512) -> np.ndarray:
    """The oracle's decoded weights [rows, cols] (bf16 bits), stored rows
    expanded in parallel chunks."""
    import concurrent.futures as cf

    import oracle

    s = p.shape
    bounds = [(b, min(s.rows, b + chunk)) for b in range(0, s.rows, chunk)]

    def part(be):
        sub = row_subset(p, np.arange(*be))
        t = sub.shape
        return oracle.expand(sub.codes, sub.scales, sub.lut, t.axis, t.T, t.L, t.k,
                             t.in_features, t.out_features)

    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return np.concatenate(list(ex.map(part, bounds)), axis=0)
