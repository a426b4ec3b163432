"""GPU parity of the fused gate/up SwiGLU entry point (trellis_gate_up_swiglu)
against the CPU oracle: h = silu(x Wg^T) * (x Wu^T), computed by the oracle in
float64 from its own decode and contraction, compared with the GPU's bf16 h
within the floored 1e-2 relative gate; repeated calls bit-identical.

Shapes: small and ragged (whole outputs), both code layouts, every M tile and
activation path of the prefill kernel, rows longer than the GEMV stages, more
rows than one persistent round, and the Qwen MLP geometry (5120 -> 17408) at
k = 4 for M = 1 and 32 with the whole output compared.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import QWEN_IN, QWEN_OUT, TOL, Dev, bf16_bits, bf16_to_f64, gate, oracle_columns, say

pytestmark = pytest.mark.gpu
CFG = synth.CONFIG_IDS
L = 12


def problems(shape, M, cfg, proj0):
    pg = synth.make_problem(shape, M, cfg, proj=proj0)
    pu = synth.make_problem(shape, M, cfg, proj=proj0 + 1)
    return pg, pu


def oracle_h(shape, pg, pu, x_bits, n_begin=0, n_end=None):
    """The oracle on the problems' codes, which synth draws row-major (the
    device copy is rewritten into the shape's layout by device_codes)."""
    s = shape
    return oracle.mlp_up_swiglu_f64(x_bits, (pg.codes, pg.scales, pg.lut),
                                    (pu.codes, pu.scales, pu.lut), s.T, s.L, s.k,
                                    s.in_features, s.out_features, n_begin, n_end)


def device_codes(T, p, shape):
    d = Dev(p, T)
    codes = d.codes
    if shape.block_interleave == 2:
        nb = shape.cols // 256
        il = oracle.interleave_blocks(p.codes, shape.rows, nb, 8 * shape.k)
        codes = torch.from_numpy(il.view(np.int32)).to("cuda")
    return d, (codes, d.scales, d.lut)


def run_swiglu(T, shape, pg, pu):
    dg, gate_ops = device_codes(T, pg, shape)
    _, up_ops = device_codes(T, pu, shape)
    x = dg.x if pg.M > 1 else dg.x.reshape(1, -1)
    h = T.gate_up_swiglu(x, gate_ops, up_ops, shape)
    torch.cuda.synchronize()
    return h, (x, gate_ops, up_ops)


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 9, 16, 17, 32])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_swiglu_small(gpu_lib, M, k):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, 1024, 300)
    pg, pu = problems(shape, M, CFG["test"], 1000 + 10 * k)
    say(f"swiglu small in=1024 out=300 k={k} M={M}")
    h, _ = run_swiglu(T, shape, pg, pu)
    assert h.shape == (M, 300)
    assert gate(bf16_to_f64(h), oracle_h(shape, pg, pu, pg.x)) <= TOL


@pytest.mark.parametrize("i,o,k,M,il", [(512, 256, 2, 1, 0), (768, 4111, 3, 1, 0),
                                        (2048, 600, 4, 1, 2), (512, 16, 3, 3, 2),
                                        (1536, 1000, 2, 12, 2), (256, 1, 4, 1, 0),
                                        (256, 1, 2, 32, 0), (12288, 300, 2, 1, 0),
                                        (32768, 40, 4, 1, 0), (256, 21000, 3, 6, 0),
                                        (512, 16, 3, 20, 2), (256, 21000, 4, 24, 0),
                                        (1024, 1, 3, 32, 0), (2048, 4111, 4, 17, 2),
                                        (768, 37, 4, 31, 0), (4096, 18500, 3, 32, 2),
                                        (768, 5000, 2, 5, 0), (1024, 5000, 4, 8, 2)])
def test_swiglu_shapes(gpu_lib, i, o, k, M, il):
    """Ragged row counts, one row, one block per row, block interleave 2, rows
    longer than the GEMV stages (12288 inputs at k = 2, 32768 at k = 4: the
    16-row-group kernel with one activation row), and more rows than one
    persistent round holds (21000). At k = 3, 4 and M > 16 gate and up rows
    share 16-row groups: one row of each per workgroup (16, 1 rows), an odd
    count per workgroup (37, 4111), and more workgroups than compute units
    (21000 and 18500 rows, more than 72 per compute unit). At 5000 rows and
    M <= 8 the last group of each workgroup is folded (two blocks per task)."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o, il)
    pg, pu = problems(shape, M, CFG["test"], 1100 + i % 97 + o % 89)
    say(f"swiglu in={i} out={o} k={k} M={M} interleave={il}")
    h, _ = run_swiglu(T, shape, pg, pu)
    assert gate(bf16_to_f64(h), oracle_h(shape, pg, pu, pg.x)) <= TOL


def test_swiglu_deterministic(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 3, 2048, 999)
    for M in (1, 7, 24):
        pg, pu = problems(shape, M, CFG["test"], 1200 + M)
        say(f"swiglu determinism M={M}")
        h, (x, g_ops, u_ops) = run_swiglu(T, shape, pg, pu)
        h2 = T.gate_up_swiglu(x, g_ops, u_ops, shape)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(h), bf16_bits(h2))


def test_swiglu_one_hot_matches_stored_weights(gpu_lib):
    """One-hot rows: g and u are single stored weights (exact in float32), so
    h = bf16(silu(wg) * wu) up to silu's float32 evaluation."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 4, 1024, 500)
    pg, pu = problems(shape, 4, CFG["test"], 1300)
    cols = [0, 255, 256, 1023]
    x = synth.one_hot_x(4, 1024, cols)
    pg = synth.Problem(shape, 4, pg.codes, pg.lut, pg.scales, x)
    say("swiglu one-hot k=4 M=4")
    h, _ = run_swiglu(T, shape, pg, pu)
    ref = oracle_h(shape, pg, pu, x)
    got = bf16_to_f64(h)
    # bf16 rounding of h plus a few float32 ulps of silu: 2^-8 relative
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -8, atol=1e-30)


@pytest.mark.parametrize("M", [1, 32])
def test_swiglu_qwen_mlp_full(gpu_lib, M):
    """The MLP geometry at k = 4 (5120 -> 17408), every output compared."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 4, QWEN_IN, QWEN_OUT)
    pg, pu = problems(shape, M, CFG["qwen_mlp"], 0)
    say(f"swiglu qwen mlp k=4 M={M} (full output)")
    h, _ = run_swiglu(T, shape, pg, pu)
    ref = oracle_columns(lambda b, e: oracle_h(shape, pg, pu, pg.x, b, e), QWEN_OUT)
    assert gate(bf16_to_f64(h).reshape(M, -1), ref) <= TOL
