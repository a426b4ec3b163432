"""The scatter entry point that allocates nothing (trellis_gemv_scatter_static:
its split-K partials in the library's static device array) against the
regular trellis_gemv_scatter with a caller workspace, through the C ABI: two
calls in a row, the second on a smaller problem, each bit-identical to the
regular call on the same inputs (same kernels, same split), and within the
oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import QWEN_IN, QWEN_OUT, TOL, Dev, bf16_bits, bf16_to_f64, gate, say

pytestmark = pytest.mark.gpu


def test_static_scatter_matches_workspace_scatter(gpu_lib):
    T = gpu_lib
    assert T.static_scratch_bytes() == 2 << 20
    # the down projection (whole bands), the up projection's shape stored on
    # axis 0 (a partial band, whose zero-filled slots the static array keeps
    # between calls), then a smaller problem
    cases = [(synth.Shape(0, 256, 12, 3, QWEN_OUT, QWEN_IN), synth.CONFIG_IDS["qwen_down_scatter"]),
             (synth.Shape(0, 256, 12, 3, QWEN_IN, QWEN_OUT), synth.CONFIG_IDS["test"]),
             (synth.Shape(0, 256, 12, 2, 300, 512), synth.CONFIG_IDS["test"])]
    for shape, cfg in cases:
        p = synth.make_problem(shape, 1, cfg, proj=77)
        say(f"static scatter in={shape.in_features} out={shape.out_features} k={shape.k}")
        d = Dev(p, T)
        x = d.x.reshape(-1)
        y_static = T.gemv_scatter_static(x, d.codes, d.scales, d.lut, shape)
        y_ws = T.gemv_scatter(x, d.codes, d.scales, d.lut, shape)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y_static), bf16_bits(y_ws))
        cols = np.arange(0, shape.out_features, 37)
        ref = oracle.fused_f64(p.x, p.codes, p.scales, p.lut, 0, 256, 12, shape.k,
                               shape.in_features, shape.out_features)
        assert gate(bf16_to_f64(y_static)[cols], ref[0, cols]) <= TOL
