"""GPU parity for the block-interleave-2 code layout (page 60 vector-expand.ts
and page 59 scatter.ts address block b of row r at (b/2)*rows*2*wpb + r*2*wpb
+ (b%2)*wpb when INTERLEAVE is set).

Interleaved inputs are built on the host by the oracle's reshape-and-transpose
(oracle.interleave_blocks), never by the HIP path. Bars:
- the HIP repack writes exactly the oracle's interleaved array, and back;
- decoded weights from interleaved codes are bit-exact against the oracle's
  expand of the same interleaved codes;
- every fused operation on interleaved codes is bit-identical to the same
  operation on the row-major codes (the layout changes addresses only, never
  the summation order) and within the output tolerance of the oracle run on
  the interleaved codes.
Small and ragged shapes are compared in full; the 5120 x 17408 workloads by
layout invariance at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import QWEN_IN, QWEN_OUT, TOL, Dev, bf16_bits, bf16_to_f64, gate, say

pytestmark = pytest.mark.gpu
CFG = synth.CONFIG_IDS
L = 12


def interleaved(p: synth.Problem) -> synth.Problem:
    s = p.shape
    nb, wpb = s.cols // s.T, s.T * s.k // 32
    codes = oracle.interleave_blocks(p.codes, s.rows, nb, wpb).reshape(p.codes.shape)
    shape = synth.Shape(s.axis, s.T, s.L, s.k, s.in_features, s.out_features, 2)
    return synth.Problem(shape, p.M, codes, p.lut, p.scales, p.x)


def run(T, d, op):
    if op == "gemv":
        y = T.gemv(d.x.reshape(-1), d.codes, d.scales, d.lut, d.shape)
    elif op == "scatter":
        y = T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, d.shape)
    else:
        y = T.prefill(d.x, d.codes, d.scales, d.lut, d.shape)
    torch.cuda.synchronize()
    return y.reshape(d.p.M, -1)


def oracle_y(p):
    s = p.shape
    return oracle.fused_f64(p.x, p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k,
                            s.in_features, s.out_features, block_interleave=s.block_interleave)


# ---------------------------------------------------------------- repack
@pytest.mark.parametrize("rows,cols", [(37, 1024), (5, 512), (300, 2048)])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_repack_writes_the_oracle_layout(gpu_lib, rows, cols, k):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, cols, rows)
    p = synth.make_problem(shape, 1, CFG["test"], proj=300 + k)
    want = oracle.interleave_blocks(p.codes, rows, cols // 256, 8 * k)
    say(f"repack rows={rows} cols={cols} k={k}")
    src = torch.from_numpy(p.codes.view(np.int32)).cuda()
    il = T.repack(src, shape, 2)
    torch.cuda.synchronize()
    assert np.array_equal(il.cpu().numpy().view(np.uint32).ravel(), want)
    back = T.repack(il, synth.Shape(1, 256, L, k, cols, rows, 2), 0)
    same = T.repack(src, shape, 0)
    torch.cuda.synchronize()
    assert torch.equal(back, src) and torch.equal(same, src)


def test_repack_qwen_down_k3(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, QWEN_OUT, QWEN_IN)
    p = synth.make_problem(shape, 1, CFG["qwen_down_scatter"])
    want = oracle.interleave_blocks(p.codes, shape.rows, shape.cols // 256, 24)
    say("repack qwen down k=3")
    src = torch.from_numpy(p.codes.view(np.int32)).cuda()
    il = T.repack(src, shape, 2)
    torch.cuda.synchronize()
    assert np.array_equal(il.cpu().numpy().view(np.uint32).ravel(), want)


# ---------------------------------------------------------------- expand
@pytest.mark.parametrize("axis,i,o", [(1, 1024, 300), (0, 37, 1024), (1, 512, 5)])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_expand_interleaved_bit_exact(gpu_lib, axis, i, o, k):
    T = gpu_lib
    p = interleaved(synth.make_problem(synth.Shape(axis, 256, L, k, i, o), 1, CFG["test"],
                                       proj=310 + k))
    s = p.shape
    say(f"expand interleaved axis={axis} in={i} out={o} k={k}")
    d = Dev(p, T)
    W = bf16_bits(T.expand(d.codes, d.scales, d.lut, s))
    ref = oracle.expand(p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k, s.in_features,
                        s.out_features, block_interleave=2)
    assert np.array_equal(W, ref)


# ---------------------------------------------------------------- fused ops
CASES = [
    ("gemv", 1, 1024, 300, 1),       # persistent GEMV kernel
    ("gemv", 1, 12288, 40, 1),       # rows longer than the GEMV's LDS: axis-1 kernel, M = 1
    ("scatter", 0, 1000, 1024, 1),
    ("scatter", 0, 37, 512, 1),
    ("prefill", 1, 1024, 300, 5),    # direct activation path
    ("prefill", 1, 1024, 300, 12),   # staged activation path
    ("prefill", 1, 1024, 300, 17),   # two M tiles
    ("prefill", 0, 300, 1024, 3),
    ("prefill", 0, 300, 1024, 20),
    ("scatter", 0, 2050, 17408, 1),   # axis 0, a partial band (136 tiles)
    ("prefill", 0, 2050, 17408, 20),
]


@pytest.mark.parametrize("op,axis,i,o,M", CASES)
@pytest.mark.parametrize("k", [2, 3, 4])
def test_fused_ops_layout_invariant(gpu_lib, op, axis, i, o, M, k):
    T = gpu_lib
    p0 = synth.make_problem(synth.Shape(axis, 256, L, k, i, o), M, CFG["test"], proj=320 + k)
    p2 = interleaved(p0)
    say(f"interleave {op} axis={axis} in={i} out={o} M={M} k={k}")
    y0 = run(T, Dev(p0, T), op)
    y2 = run(T, Dev(p2, T), op)
    assert np.array_equal(bf16_bits(y0), bf16_bits(y2))
    assert gate(bf16_to_f64(y2), oracle_y(p2)) <= TOL


@pytest.mark.parametrize("op,k,M", [("gemv", 2, 1), ("gemv", 4, 1), ("scatter", 3, 1),
                                    ("prefill", 2, 5), ("prefill", 3, 16), ("prefill", 4, 32)])
def test_qwen_workloads_layout_invariant(gpu_lib, op, k, M):
    """Full-size workloads in the benchmark's launch configuration: the
    interleaved layout gives the row-major layout's bits."""
    T = gpu_lib
    axis = 0 if op == "scatter" else 1
    shape = (synth.Shape(0, 256, L, k, QWEN_OUT, QWEN_IN) if axis == 0
             else synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT))
    p0 = synth.make_problem(shape, M, CFG["test"], proj=330 + k)
    p2 = interleaved(p0)
    say(f"interleave qwen {op} k={k} M={M}")
    y0 = run(T, Dev(p0, T), op)
    y2 = run(T, Dev(p2, T), op)
    assert np.array_equal(bf16_bits(y0), bf16_bits(y2))
