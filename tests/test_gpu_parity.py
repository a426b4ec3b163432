"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: decoded weights bit-exact; one-hot activations and integer codebooks
bit-exact (a single product, or sums exact in float32, leave one correct bf16
answer); random activations within max relative error 1e-2 (the floored gate
in helpers.gate); repeated calls bit-identical. Sizes: tiny and ragged shapes
compared in full; the 5120 x 17408 shapes compared in full too (the oracle
runs column or row chunks on a thread pool), in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import (QWEN_IN, QWEN_OUT, TOL, Dev, bf16_bits, bf16_to_f64, gate, oracle_W_full,
                     oracle_y_full, row_subset, say, with_x)

pytestmark = pytest.mark.gpu
CFG = synth.CONFIG_IDS
L = 12


def oracle_y(p, n_begin=0, n_end=None):
    s = p.shape
    return oracle.fused_f64(p.x, p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k,
                            s.in_features, s.out_features, n_begin, n_end,
                            block_interleave=s.block_interleave)


def oracle_W(p):
    s = p.shape
    return oracle.expand(p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k, s.in_features,
                         s.out_features)


def run(T, d, op=None):
    """Dispatch by op: gemv (axis 1, M=1), scatter (axis 0, M=1) or prefill."""
    if op == "gemv":
        y = T.gemv(d.x.reshape(-1), d.codes, d.scales, d.lut, d.shape)
    elif op == "scatter":
        y = T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, d.shape)
    else:
        y = T.prefill(d.x, d.codes, d.scales, d.lut, d.shape)
    torch.cuda.synchronize()
    return y.reshape(d.p.M, -1)


# --------------------------------------------------------------- expand
@pytest.mark.parametrize("axis,i,o", [(1, 512, 256), (1, 768, 300), (0, 300, 512), (0, 37, 256)])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_expand_bit_exact_small(gpu_lib, axis, i, o, k):
    T = gpu_lib
    shape = synth.Shape(axis, 256, L, k, i, o)
    p = synth.make_problem(shape, 1, CFG["test"], proj=100 + k)
    say(f"expand small axis={axis} in={i} out={o} k={k}")
    d = Dev(p, T)
    W = bf16_bits(T.expand(d.codes, d.scales, d.lut, shape))
    assert np.array_equal(W, oracle_W(p))


@pytest.mark.parametrize("k", [2, 3, 4])
def test_expand_bit_exact_qwen_full(gpu_lib, k):
    """Every decoded weight of the 17408 x 5120 matrix, bit for bit."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT)
    p = synth.make_problem(shape, 1, CFG["qwen_up_gemv"])
    say(f"expand qwen-up k={k} (every weight)")
    d = Dev(p, T)
    W = bf16_bits(T.expand(d.codes, d.scales, d.lut, shape))
    assert np.array_equal(W, oracle_W_full(p))


# ----------------------------------------------------------------- GEMV
@pytest.mark.parametrize("i,o", [(512, 256), (768, 300), (256, 17), (1024, 1), (12288, 300),
                                 (32768, 40)])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_gemv_small(gpu_lib, i, o, k):
    """Small and ragged shapes; 12288 and 32768 inputs exceed the activations
    the persistent kernel stages in LDS (for k = 2, resp. all k) and take the
    general axis-1 kernel."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o)
    p = synth.make_problem(shape, 1, CFG["tiny_gemv"] if (i, o) == (512, 256) else CFG["test"])
    say(f"gemv small in={i} out={o} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T), op="gemv"))
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("i,o", [(QWEN_IN, 80000), (46 * 256, 30000)])
@pytest.mark.parametrize("k", [2, 4])
def test_gemv_rows_in_several_chunks(gpu_lib, i, o, k):
    """More rows per workgroup than the unit partials the persistent kernel
    holds in LDS at once (what the staged activations leave: 5552 units, i.e.
    277 rows of 20 blocks, or 2120 units, 46 rows of 46 blocks), so each
    workgroup runs several row chunks: 313 rows of 20 blocks (two chunks) and
    118 rows of 46 blocks, the longest rows the kernel stages (three).
    Checked on rows spread over the range."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o)
    p = synth.make_problem(shape, 1, CFG["test"], proj=800 + k)
    say(f"gemv in={i} out={o} k={k} (several row chunks per workgroup)")
    y = bf16_to_f64(run(T, Dev(p, T), op="gemv"))
    assert gate(y, oracle_y_full(p)) <= TOL


@pytest.mark.parametrize("k", [2, 3, 4])
def test_gemv_qwen_full(gpu_lib, k):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT)
    p = synth.make_problem(shape, 1, CFG["qwen_up_gemv"])
    say(f"gemv qwen-up k={k} (whole output)")
    y = bf16_to_f64(run(T, Dev(p, T), op="gemv"))
    assert gate(y, oracle_y_full(p)) <= TOL


@pytest.mark.parametrize("k", [2, 3, 4])
def test_gemv_one_hot_columns_bit_exact(gpu_lib, k):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT)
    p = synth.make_problem(shape, 1, CFG["qwen_up_gemv"])
    d = Dev(p, T)
    W = oracle_W_full(p)
    for col in (0, 1, 255, 256, 2047, 4000, QWEN_IN - 1):
        say(f"gemv one-hot k={k} col={col}")
        x = synth.one_hot_x(1, QWEN_IN, [col])
        d.x.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        y = bf16_bits(run(T, d, op="gemv"))[0]
        assert np.array_equal(y, W[:, col])


@pytest.mark.parametrize("k", [2, 3, 4])
def test_gemv_integer_codebook_bit_exact(gpu_lib, k):
    """Integer codebook, scales in {0.5, 1, 2}, integer x: every partial sum is
    exact in float32, so the bf16 output is unique whatever the order."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, 2048)
    g = np.random.default_rng(7 + k)
    p0 = synth.make_problem(shape, 1, CFG["test"], proj=200 + k)
    xi = g.integers(-3, 4, (1, QWEN_IN)).astype(np.float32)
    p = synth.Problem(shape, 1, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say(f"gemv integer codebook k={k}")
    y = bf16_bits(run(T, Dev(p, T), op="gemv"))
    exact = oracle_y(p)
    assert np.all(np.abs(exact) < 2**24)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


def test_gemv_deterministic(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 3, QWEN_IN, QWEN_OUT)
    d = Dev(synth.make_problem(shape, 1, CFG["qwen_up_gemv"]), T)
    say("gemv determinism k=3")
    a = bf16_bits(run(T, d, op="gemv"))
    b = bf16_bits(run(T, d, op="gemv"))
    assert np.array_equal(a, b)


# -------------------------------------------------------------- scatter
@pytest.mark.parametrize("i,o", [(512, 256), (1000, 512), (17, 256), (4096, 768)])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_scatter_small(gpu_lib, i, o, k):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, k, i, o)
    p = synth.make_problem(shape, 1, CFG["test"], proj=300 + k)
    say(f"scatter small in={i} out={o} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T), op="scatter"))
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("k", [3, 2, 4])
def test_scatter_qwen_down_full(gpu_lib, k):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, k, QWEN_OUT, QWEN_IN)
    p = synth.make_problem(shape, 1, CFG["qwen_down_scatter"])
    say(f"scatter qwen-down k={k} (whole output)")
    y = bf16_to_f64(run(T, Dev(p, T), op="scatter"))
    assert gate(y, oracle_y_full(p)) <= TOL


def test_scatter_one_hot_rows_bit_exact(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, QWEN_OUT, QWEN_IN)
    p = synth.make_problem(shape, 1, CFG["qwen_down_scatter"])
    d = Dev(p, T)
    for r in (0, 135, 136, 9000, QWEN_OUT - 1):
        say(f"scatter one-hot row={r}")
        x = synth.one_hot_x(1, QWEN_OUT, [r])
        d.x.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        y = bf16_bits(run(T, d, op="scatter"))[0]
        assert np.array_equal(y, oracle_W(row_subset(p, np.array([r])))[0])


def test_scatter_integer_codebook_bit_exact(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, 4096, 1024)
    g = np.random.default_rng(77)
    p0 = synth.make_problem(shape, 1, CFG["test"], proj=400)
    xi = g.integers(-3, 4, (1, shape.in_features)).astype(np.float32)
    p = synth.Problem(shape, 1, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say("scatter integer codebook k=3")
    y = bf16_bits(run(T, Dev(p, T), op="scatter"))
    exact = oracle_y(p)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("i,o,M,k", [(2050, 17408, 1, 3), (2050, 17408, 20, 4), (320, 17408, 1, 2)])
def test_axis0_partial_band_integer_codebook_bit_exact(gpu_lib, i, o, M, k):
    """The finer axis-0 split (a partial band, a tile's last ranges in two
    workgroups, zero-filled second slots) with an integer codebook, scales in
    {0.5, 1, 2} and small-integer activations: every partial and sum is exact
    in float32, so the output is the exact result rounded once to bf16."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, k, i, o)
    g = np.random.default_rng(78 + M + k)
    p0 = synth.make_problem(shape, M, CFG["test"], proj=401)
    xi = g.integers(-3, 4, (M, shape.in_features)).astype(np.float32)
    p = synth.Problem(shape, M, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say(f"axis0 partial band integer codebook in={i} out={o} M={M} k={k}")
    d = Dev(p, T)
    y = bf16_bits(run(T, d, op="scatter") if M == 1 else run(T, d)).reshape(M, -1)
    exact = oracle_y_full(p)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("M", [1, 3, 20])
def test_axis0_fewer_rows_than_splits(gpu_lib, M):
    """37 input rows: two 32-row steps in two row ranges, so most waves of a
    workgroup have no step, and an odd row count (the element-wise activation
    path)."""
    T = gpu_lib
    k = 2 + M % 3
    shape = synth.Shape(0, 256, L, k, 37, 512)
    p = synth.make_problem(shape, M, CFG["test"], proj=900 + M)
    say(f"axis0 in=37 out=512 M={M} k={k}")
    d = Dev(p, T)
    y = run(T, d, op="scatter") if M == 1 else run(T, d)
    assert gate(bf16_to_f64(y), oracle_y(p)) <= TOL


@pytest.mark.parametrize("i,o,M,k", [(5120, 17408, 1, 2), (5120, 17408, 32, 4), (2050, 17408, 20, 3),
                                     (1000, 20480, 1, 4), (96, 17408, 3, 3), (4099, 1280, 1, 3),
                                     (320, 17408, 1, 3), (640, 24320, 4, 2), (4096, 11520, 1, 4)])
def test_axis0_partial_band(gpu_lib, i, o, M, k):
    """Shapes where one workgroup per (band of 8 row ranges, tile) would leave
    a quarter or more of the compute units idle, so every tile's rows are cut
    into more ranges and the last band's ranges of several tiles share
    workgroups (a tile's may span two): 136 tiles in 15 ranges (M = 1, and 32
    in two M tiles), 2050 ragged rows (element-wise activation loads) in 15,
    160 tiles in 12, 96 rows = 3 ranges on 2 waves per workgroup (one range per
    tile in the last band), 320 rows = 10 ranges on 6 waves per workgroup, 190
    tiles in 10 ranges (a last band of 2 per tile), 90 tiles in 22 (6 per
    tile); and 4099 x 10 tiles, which keeps whole bands."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, k, i, o)
    p = synth.make_problem(shape, M, CFG["test"], proj=950 + M + k)
    say(f"axis0 partial band in={i} out={o} M={M} k={k}")
    d = Dev(p, T)
    y = run(T, d, op="scatter") if M == 1 else run(T, d)
    ref = oracle_y_full(p) if o > 4096 else oracle_y(p)
    assert gate(bf16_to_f64(y), ref) <= TOL


def test_scatter_deterministic(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, QWEN_OUT, QWEN_IN)
    d = Dev(synth.make_problem(shape, 1, CFG["qwen_down_scatter"]), T)
    say("scatter determinism k=3")
    assert np.array_equal(bf16_bits(run(T, d, op="scatter")), bf16_bits(run(T, d, op="scatter")))


# -------------------------------------------------------------- prefill
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 17, 32])
@pytest.mark.parametrize("axis", [1, 0])
def test_prefill_small(gpu_lib, M, axis):
    T = gpu_lib
    k = 2 + M % 3
    shape = synth.Shape(axis, 256, L, k, 768 if axis else 1000, 300 if axis else 512)
    p = synth.make_problem(shape, M, CFG["test"], proj=500 + axis)
    say(f"prefill small axis={axis} M={M} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert y.shape == (M, shape.out_features)
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("M", [3, 20])
def test_prefill_axis1_more_rows_than_persistent_grid(gpu_lib, M):
    """25000 output rows exceed 80 rows per workgroup on every compute unit:
    the axis-1 kernel then launches workgroups in rounds. Two blocks per row
    leave most waves of a workgroup without tasks."""
    T = gpu_lib
    k = 2 + M % 3
    shape = synth.Shape(1, 256, L, k, 512, 25000)
    p = synth.make_problem(shape, M, CFG["test"], proj=600 + M)
    say(f"prefill axis=1 in=512 out=25000 M={M} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("M", [5, 8, 16, 32])
def test_prefill_qwen_up_full(gpu_lib, M, k):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT)
    p = synth.make_problem(shape, M, CFG["qwen_up_prefill"])
    say(f"prefill qwen-up M={M} k={k} (whole output)")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y_full(p)) <= TOL


def test_prefill_one_hot_rows_bit_exact(gpu_lib):
    """Each activation row one-hot: output row m is column cols[m] of W."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 4, QWEN_IN, QWEN_OUT)
    cols = [0, 17, 255, 256, 1023, 2500, 5119, 64, 128, 3, 777, 4096, 300, 301, 2, 1,
            4000, 4001, 11, 12, 13, 14, 15, 16, 2047, 2048, 3071, 3072, 5000, 5001, 5002, 999]
    p0 = synth.make_problem(shape, 32, CFG["qwen_up_prefill"])
    p = with_x(p0, synth.one_hot_x(32, QWEN_IN, cols))
    say("prefill one-hot M=32 k=4")
    y = bf16_bits(run(T, Dev(p, T)))
    W = oracle_W_full(p)
    for m, c in enumerate(cols):
        assert np.array_equal(y[m], W[:, c]), (m, c)


# ------------------------------------- axis 1, up to 4 rows in the GEMV's unit mapping
@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("N", [16, 31, 300, 4111])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_rows_kernel_ragged(gpu_lib, N, M, k):
    """Up to 4 activation rows take the GEMV's unit mapping with M outputs per
    unit (at k = 3, 4 on the codebook copies when the partials fit in one
    chunk): one workgroup of exactly 16 rows, one of 31, workgroups of 16-17
    rows (a step can straddle a block edge right after entering a block), and
    4111 rows over every compute unit. 5 and 8 rows take the 16-row-group
    kernel with directly loaded activations."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, 1024, N)
    p = synth.make_problem(shape, M, CFG["test"], proj=700 + M)
    say(f"rows kernel in=1024 out={N} M={M} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y(p)) <= TOL


# ------------------------------------- axis 1, folded last group (M <= 8)
FOLD_CASES = [(768, 5000, 2, 5, 0),    # 19-20 rows per workgroup: 3-4 rows folded; 3 blocks
              (1024, 5000, 3, 8, 0),   # 4 blocks
              (2048, 4500, 4, 7, 2),   # 17-18 rows: 1-2 rows folded; interleaved codes
              (1280, 17000, 2, 6, 0),  # 66-67 rows: four full groups and 2-3 rows; 5 blocks
              (256, 4400, 3, 8, 0),    # one block: the folded task's second half is empty
              (512, 6000, 4, 5, 2),    # 23-24 rows: 7-8 rows folded
              (768, 6200, 2, 8, 0)]    # 24-25 rows: a last group of 8 rows folds, of 9 does not


@pytest.mark.parametrize("i,o,k,M,il", FOLD_CASES)
def test_prefill_folded_last_group(gpu_lib, i, o, k, M, il):
    """With directly loaded activations and M <= 8, a last 16-row group of at
    most 8 rows decodes two blocks per task (A and B each hold two blocks'
    8 rows): odd and even block counts, one block, 1 to 8 folded rows, and
    workgroups on both sides of the 8-row limit."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o, il)
    p = synth.make_problem(shape, M, CFG["test"], proj=1700 + M + k)
    say(f"prefill folded in={i} out={o} k={k} M={M} interleave={il}")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("i,o,k,M", [(768, 5000, 2, 6), (256, 4400, 3, 8), (1280, 17000, 4, 5)])
def test_prefill_folded_integer_codebook_bit_exact(gpu_lib, i, o, k, M):
    """The folded group with an integer codebook and integer activations: both
    blocks' quarters of every tile are exact, so each output is the unique
    bf16 of the exact sum; a lane past the last block must add zero."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o)
    g = np.random.default_rng(90 + M + k)
    p0 = synth.make_problem(shape, M, CFG["test"], proj=1750 + M)
    xi = g.integers(-3, 4, (M, shape.in_features)).astype(np.float32)
    p = synth.Problem(shape, M, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say(f"prefill folded integer codebook in={i} out={o} k={k} M={M}")
    y = bf16_bits(run(T, Dev(p, T)))
    exact = oracle_y(p)
    assert np.all(np.abs(exact) < 2**24)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("i", [256, 512])
@pytest.mark.parametrize("M", [3, 7])
def test_rows_kernel_one_or_two_blocks_per_row(gpu_lib, i, M):
    """One block per row (no step can straddle) and two (the interleaved
    layout coincides with the row-major one); M = 3 in the GEMV's unit
    mapping, M = 7 in 16-row groups."""
    T = gpu_lib
    k = 3
    for il in (0, 2):
        if il and i // 256 % 2:
            continue
        shape = synth.Shape(1, 256, L, k, i, 300, il)
        p = synth.make_problem(shape, M, CFG["test"], proj=740 + M)
        say(f"rows kernel in={i} out=300 M={M} k={k} interleave={il}")
        y = bf16_to_f64(run(T, Dev(p, T)))
        ref = oracle.fused_f64(p.x, p.codes, p.scales, p.lut, 1, 256, L, k, i, 300,
                               block_interleave=il)
        assert gate(y, ref) <= TOL


def test_rows_kernel_two_chunks_k4(gpu_lib):
    """Rows of 256 blocks at M = 4: beside the codebook copies fewer than 16
    rows' partials fit, so the kernel reads the single codebook, beside which
    32 rows' partials fit: 40-row workgroups run two chunks of 20 rows."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 4, 65536, 10240)
    p = synth.make_problem(shape, 4, CFG["test"], proj=710)
    say("rows kernel in=65536 out=10240 M=4 k=4")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y_full(p)) <= TOL


def test_rows_kernel_falls_back_when_partials_do_not_fit(gpu_lib):
    """128 blocks per row at M = 4, k = 2: fewer than 16 rows' partials fit
    beside the pair table, so the call takes the 16-row-group kernel."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 2, 32768, 300)
    p = synth.make_problem(shape, 4, CFG["test"], proj=720)
    say("rows kernel fallback in=32768 out=300 M=4 k=2")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y(p)) <= TOL


@pytest.mark.parametrize("M", [4, 8])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_rows_kernel_one_hot_bit_exact(gpu_lib, k, M):
    """Four one-hot activation rows (the GEMV's unit mapping) and eight
    (16-row groups, activations loaded directly) at the Qwen-up shape: each
    output row is one stored column exactly."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT)
    cols = [0, 255, 256, 2047, 2048, 4095, 5119, 1000][:M]
    p0 = synth.make_problem(shape, M, CFG["qwen_up_prefill"], proj=730)
    p = with_x(p0, synth.one_hot_x(M, QWEN_IN, cols))
    say(f"rows kernel one-hot M={M} k={k}")
    y = bf16_bits(run(T, Dev(p, T)))
    W = oracle_W_full(p)
    for m, c in enumerate(cols):
        assert np.array_equal(y[m], W[:, c]), (m, c)


@pytest.mark.parametrize("M", [5, 8, 32])
def test_prefill_axis0_qwen_down_full(gpu_lib, M):
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 4, QWEN_OUT, QWEN_IN)
    p = synth.make_problem(shape, M, CFG["qwen_mlp"], proj=2)
    say(f"prefill axis0 qwen-down M={M} k=4 (whole output)")
    y = bf16_to_f64(run(T, Dev(p, T)))
    assert gate(y, oracle_y_full(p)) <= TOL


def test_axis0_workspace_reused_across_shapes(gpu_lib):
    """One workspace, sized for the largest call, serves a sequence of axis-0
    calls of different shapes and batch sizes; stale contents do not leak."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, 1000, 768)
    big = synth.Shape(0, 256, L, 2, 4000, 1280)
    ws = torch.full((T.workspace_bytes(big, 32, T.OP_PREFILL) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda:0")
    for sh, M in ((shape, 1), (big, 32), (shape, 8), (big, 1), (shape, 32), (shape, 1)):
        p = synth.make_problem(sh, M, CFG["test"], proj=700 + M + sh.k)
        say(f"axis0 reused workspace in={sh.in_features} out={sh.out_features} M={M} k={sh.k}")
        d = Dev(p, T)
        if M == 1:
            y = T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, sh, workspace=ws)
        else:
            y = T.prefill(d.x, d.codes, d.scales, d.lut, sh, workspace=ws)
        torch.cuda.synchronize()
        assert gate(bf16_to_f64(y.reshape(M, -1)), oracle_y(p)) <= TOL


@pytest.mark.parametrize("fill", [0x00, 0xFF])
def test_axis0_workspace_contents_do_not_matter(gpu_lib, fill):
    """Workspace bytes all zero or all ones on entry, then the same call five
    times in a row on it (each call leaves its flags behind for the next):
    every result bit-identical and within tolerance of the oracle."""
    T = gpu_lib
    sh = synth.Shape(0, 256, L, 3, 3000, 1024)
    for M in (1, 4, 20):
        p = synth.make_problem(sh, M, CFG["test"], proj=760 + M)
        d = Dev(p, T)
        nbytes = T.workspace_bytes(sh, M, T.OP_PREFILL)
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda:0").view(torch.float32)
        say(f"axis0 workspace filled {fill:#04x} M={M}")
        ys = []
        for _ in range(5):
            y = (T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, sh, workspace=ws)
                 if M == 1 else T.prefill(d.x, d.codes, d.scales, d.lut, sh, workspace=ws))
            ys.append(bf16_bits(y.reshape(M, -1)).copy())
        torch.cuda.synchronize()
        assert all(np.array_equal(ys[0], v) for v in ys[1:])
        assert gate(bf16_to_f64(y.reshape(M, -1)), oracle_y(p)) <= TOL


def test_prefill_deterministic(gpu_lib):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 2, QWEN_IN, QWEN_OUT)
    d = Dev(synth.make_problem(shape, 32, CFG["qwen_up_prefill"]), T)
    say("prefill determinism M=32 k=2")
    assert np.array_equal(bf16_bits(run(T, d)), bf16_bits(run(T, d)))


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("axis,M", [(1, 3), (1, 6), (1, 12), (1, 24), (0, 1), (0, 4), (0, 20)])
def test_prefill_integer_codebook_bit_exact(gpu_lib, axis, M, k):
    """Integer codebook, scales in {0.5, 1, 2}, integer activations: every
    partial sum is exact in float32, so the bf16 output is unique whatever the
    summation order. Covers each axis-1 path (the GEMV-mapped kernel, directly
    loaded and LDS-staged activations, two M tiles) and axis 0."""
    T = gpu_lib
    shape = synth.Shape(axis, 256, L, k, 1024 if axis else 1000, 600 if axis else 512)
    g = np.random.default_rng(50 + 10 * M + k + axis)
    p0 = synth.make_problem(shape, M, CFG["test"], proj=800 + M)
    xi = g.integers(-3, 4, (M, shape.in_features)).astype(np.float32)
    p = synth.Problem(shape, M, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say(f"prefill integer codebook axis={axis} M={M} k={k}")
    y = bf16_bits(run(T, Dev(p, T)))
    exact = oracle_y(p)
    assert np.all(np.abs(exact) < 2**24)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


@pytest.mark.parametrize("axis,M,k", [(1, 4, 2), (1, 7, 3), (0, 8, 3)])
def test_small_batch_deterministic(gpu_lib, axis, M, k):
    """The GEMV-mapped axis-1 kernel and the axis-0 prefill give the same bits
    on repeated calls."""
    T = gpu_lib
    shape = (synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT) if axis
             else synth.Shape(0, 256, L, k, QWEN_OUT, QWEN_IN))
    d = Dev(synth.make_problem(shape, M, CFG["test"], proj=820 + M), T)
    say(f"determinism axis={axis} M={M} k={k}")
    assert np.array_equal(bf16_bits(run(T, d)), bf16_bits(run(T, d)))


def test_prefill_axis0_one_hot_bit_exact(gpu_lib):
    """Axis 0, eight one-hot activation rows: output row m is stored row
    cols[m] of W exactly."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, 2000, 1024)
    cols = [0, 1, 7, 8, 999, 1000, 1998, 1999]
    p0 = synth.make_problem(shape, 8, CFG["test"], proj=830)
    p = with_x(p0, synth.one_hot_x(8, 2000, cols))
    say("prefill axis0 one-hot M=8 k=3")
    y = bf16_bits(run(T, Dev(p, T)))
    W = oracle_W(p)
    for m, r in enumerate(cols):
        assert np.array_equal(y[m], W[r]), (m, r)


# ------------------------------------------------------ MLP (k=4, M=1/32)
@pytest.mark.parametrize("M", [1, 32])
def test_mlp_projections_full(gpu_lib, M):
    """Gate and up (axis 1) and down (axis 0), each with its own codebook."""
    T = gpu_lib
    for proj, axis in ((0, 1), (1, 1), (2, 0)):
        shape = (synth.Shape(1, 256, L, 4, QWEN_IN, QWEN_OUT) if axis
                 else synth.Shape(0, 256, L, 4, QWEN_OUT, QWEN_IN))
        p = synth.make_problem(shape, M, CFG["qwen_mlp"], proj=proj)
        say(f"mlp proj={proj} axis={axis} M={M}")
        d = Dev(p, T)
        op = None if M > 1 else ("gemv" if axis else "scatter")
        y = bf16_to_f64(run(T, d, op=op))
        assert gate(y, oracle_y_full(p)) <= TOL


# ------------------------------------------------------------- HIP graphs
def test_graph_capture_replays_match_eager(gpu_lib):
    """The entry points enqueue only kernels (no allocation, memset or host
    sync on the compute path), so a sequence of them can be captured into a
    HIP graph. Each replay, with eager work and synchronisation in between,
    must reproduce the eager results bit for bit."""
    T = gpu_lib
    up = synth.Shape(1, 256, L, 2, 1024, 600)
    down = synth.Shape(0, 256, L, 3, 600, 768)
    pu = synth.make_problem(up, 1, CFG["test"], proj=950)
    pp = synth.make_problem(up, 5, CFG["test"], proj=951)
    pd = synth.make_problem(down, 1, CFG["test"], proj=952)
    du, dp, dd = Dev(pu, T), Dev(pp, T), Dev(pd, T)
    ws = torch.zeros(T.workspace_bytes(down, 1, T.OP_GEMV_SCATTER) // 4, dtype=torch.float32,
                     device="cuda:0")
    y1 = torch.empty(600, dtype=torch.bfloat16, device="cuda:0")
    y2 = torch.empty((5, 600), dtype=torch.bfloat16, device="cuda:0")
    y3 = torch.empty(768, dtype=torch.bfloat16, device="cuda:0")

    y4 = torch.empty((5, 600), dtype=torch.bfloat16, device="cuda:0")
    y5 = torch.empty(768, dtype=torch.bfloat16, device="cuda:0")
    y6 = torch.empty(600, dtype=torch.bfloat16, device="cuda:0")

    def step(stream):
        T.gemv(du.x.reshape(-1), du.codes, du.scales, du.lut, up, y=y1, stream=stream)
        T.prefill(dp.x, dp.codes, dp.scales, dp.lut, up, y=y2, stream=stream)
        T.gemv_scatter(dd.x.reshape(-1), dd.codes, dd.scales, dd.lut, down, workspace=ws,
                       y=y3, stream=stream)
        T.gate_up_swiglu(dp.x, (dp.codes, dp.scales, dp.lut), (du.codes, du.scales, du.lut), up,
                         h=y4, stream=stream)
        T.gemv_scatter_static(dd.x.reshape(-1), dd.codes, dd.scales, dd.lut, down, y=y5,
                              stream=stream)
        T.gate_up_swiglu(du.x, (du.codes, du.scales, du.lut), (dp.codes, dp.scales, dp.lut), up,
                         h=y6, stream=stream)

    say("graph capture: gemv + prefill + scatter + swiglu + static scatter")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.synchronize()
    ys = (y1, y2, y3, y4, y5, y6)
    ref = [bf16_bits(y.clone()) for y in ys]
    assert np.array_equal(ref[4], ref[2])   # the static scatter matches the workspace one
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, y in zip(ref, ys):
            assert np.array_equal(bf16_bits(y), r), rep
    assert gate(bf16_to_f64(y1.reshape(1, -1)), oracle_y(pu)) <= TOL


# ------------------------------------------------------------ degenerate cases
def exact_problem(shape, M, codes, seed):
    """Integer codebook, scales in {0.5, 1, 2}, activations in -3..3: every
    product and partial sum is exact in float32, so each bf16 output has one
    correct value whatever the summation order."""
    g = np.random.default_rng(seed)
    xi = g.integers(-3, 4, (M, shape.in_features)).astype(np.float32)
    return synth.Problem(shape, M, codes, synth.integer_lut(),
                         g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                         synth.to_bf16_bits(xi))


@pytest.mark.parametrize("word", [0x00000000, 0xFFFFFFFF, 0x55555555])
@pytest.mark.parametrize("op,axis,M,k", [("gemv", 1, 1, 2), ("gemv", 1, 1, 4), ("scatter", 0, 1, 3),
                                         (None, 1, 3, 3), (None, 1, 12, 4), (None, 1, 32, 2),
                                         (None, 0, 8, 4)])
def test_constant_code_words_bit_exact(gpu_lib, word, op, axis, M, k):
    """Every code word equal: all windows of a block hold one value (0, 0xFFF,
    or a fixed pattern), so every row decodes to one repeated weight."""
    T = gpu_lib
    shape = synth.Shape(axis, 256, L, k, 1024, 768)
    codes = np.full((shape.rows, shape.words_per_row), word, dtype=np.uint32)
    p = exact_problem(shape, M, codes, seed=word % 1000 + 7 * M + k)
    say(f"constant words {word:#010x} op={op or 'prefill'} axis={axis} M={M} k={k}")
    y = bf16_bits(run(T, Dev(p, T), op=op))
    assert np.array_equal(y, synth.to_bf16_bits(oracle_y(p).astype(np.float32)))


@pytest.mark.parametrize("op,axis,i,o,M,k", [("gemv", 1, 256, 1, 1, 2), ("gemv", 1, 256, 1, 1, 3),
                                             ("scatter", 0, 1, 256, 1, 3), ("scatter", 0, 1, 256, 1, 2),
                                             (None, 1, 256, 1, 32, 4), (None, 1, 256, 17, 3, 3),
                                             (None, 0, 1, 256, 32, 2), (None, 0, 9, 256, 17, 4)])
def test_minimal_shapes(gpu_lib, op, axis, i, o, M, k):
    """One block per row, a single output row, a single stored row."""
    T = gpu_lib
    p = synth.make_problem(synth.Shape(axis, 256, L, k, i, o), M, CFG["test"], proj=1200 + i + o)
    say(f"minimal op={op or 'prefill'} axis={axis} in={i} out={o} M={M} k={k}")
    y = bf16_to_f64(run(T, Dev(p, T), op=op))
    assert gate(y, oracle_y(p)) <= TOL


# ------------------------------------------------------------ dual GEMV
def dual_case(T, shape, proj, check_oracle=True):
    """gate/up pair sharing x: bit-identical to two trellis_gemv calls, and
    within tolerance of the oracle on each projection."""
    pa = synth.make_problem(shape, 1, CFG["test"], proj=proj)
    pb = with_x(synth.make_problem(shape, 1, CFG["test"], proj=proj + 1), pa.x)
    da, db = Dev(pa, T), Dev(pb, T)
    x = da.x.reshape(-1)
    ya, yb = T.gemv_dual(x, (da.codes, da.scales, da.lut), (db.codes, db.scales, db.lut), da.shape)
    ra = T.gemv(x, da.codes, da.scales, da.lut, da.shape)
    rb = T.gemv(x, db.codes, db.scales, db.lut, db.shape)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(ya), bf16_bits(ra))
    assert np.array_equal(bf16_bits(yb), bf16_bits(rb))
    return pa, pb, ya.reshape(1, -1), yb.reshape(1, -1)


@pytest.mark.parametrize("i,o,k,il", [(512, 256, 2, 0), (768, 300, 3, 0), (1024, 20, 4, 0),
                                      (4096, 4111, 2, 2), (2048, 1000, 3, 2),
                                      (256, 1, 2, 0), (256, 1, 4, 0), (512, 1, 3, 2)])
def test_gemv_dual_small(gpu_lib, i, o, k, il):
    """Ragged row counts, both layouts, and one output row (one workgroup per
    projection)."""
    T = gpu_lib
    say(f"gemv_dual in={i} out={o} k={k} interleave={il}")
    pa, pb, ya, yb = dual_case(T, synth.Shape(1, 256, L, k, i, o, il), 1100 + k)
    assert gate(bf16_to_f64(ya), oracle_y(pa)) <= TOL
    assert gate(bf16_to_f64(yb), oracle_y(pb)) <= TOL


@pytest.mark.parametrize("k", [2, 3, 4])
def test_gemv_dual_qwen_full(gpu_lib, k):
    T = gpu_lib
    say(f"gemv_dual qwen-up k={k} (whole outputs)")
    pa, pb, ya, yb = dual_case(T, synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT), 1110 + k)
    assert gate(bf16_to_f64(ya), oracle_y_full(pa)) <= TOL
    assert gate(bf16_to_f64(yb), oracle_y_full(pb)) <= TOL


def test_gemv_dual_long_rows(gpu_lib):
    """Rows too long to stage in LDS: the two projections run one after the other."""
    T = gpu_lib
    say("gemv_dual in=2^16 out=40 k=3")
    pa, pb, ya, yb = dual_case(T, synth.Shape(1, 256, L, 3, 1 << 16, 40), 1120)
    assert gate(bf16_to_f64(ya), oracle_y(pa)) <= TOL
    assert gate(bf16_to_f64(yb), oracle_y(pb)) <= TOL


# ------------------------------------------------------------ dual prefill
def prefill_dual_case(T, shape, M, proj):
    """gate/up pair sharing x [M][in]: each projection within tolerance of the
    oracle and of its own trellis_prefill call; a second dual call repeats the
    first bit for bit."""
    pa = synth.make_problem(shape, M, CFG["test"], proj=proj)
    pb = with_x(synth.make_problem(shape, M, CFG["test"], proj=proj + 1), pa.x)
    da, db = Dev(pa, T), Dev(pb, T)
    ya, yb = T.prefill_dual(da.x, (da.codes, da.scales, da.lut), (db.codes, db.scales, db.lut),
                            da.shape)
    ya2, yb2 = T.prefill_dual(da.x, (da.codes, da.scales, da.lut),
                              (db.codes, db.scales, db.lut), da.shape)
    ra = T.prefill(da.x, da.codes, da.scales, da.lut, da.shape)
    rb = T.prefill(da.x, db.codes, db.scales, db.lut, db.shape)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(ya), bf16_bits(ya2))
    assert np.array_equal(bf16_bits(yb), bf16_bits(yb2))
    assert gate(bf16_to_f64(ya), bf16_to_f64(ra)) <= TOL
    assert gate(bf16_to_f64(yb), bf16_to_f64(rb)) <= TOL
    return pa, pb, bf16_to_f64(ya), bf16_to_f64(yb)


@pytest.mark.parametrize("i,o,k,M,il", [(512, 300, 2, 5, 0), (768, 4111, 3, 8, 0),
                                        (1024, 1000, 4, 16, 0), (2048, 700, 2, 12, 0),
                                        (4096, 1000, 3, 6, 2), (512, 17, 4, 9, 0),
                                        (256, 1, 2, 7, 0), (512, 300, 3, 3, 0),
                                        (1024, 4111, 2, 2, 0), (512, 300, 4, 20, 0),
                                        (1024, 1000, 2, 32, 0), (2048, 4111, 3, 17, 2),
                                        (768, 300, 2, 1, 0), (1024, 5000, 2, 8, 0),
                                        (1024, 4800, 3, 5, 2)])
def test_prefill_dual_small(gpu_lib, i, o, k, M, il):
    """One shared launch for 2..32 rows (direct and staged activations, one
    and two M tiles, ragged and single-row groups, interleaved codes, a folded
    last group at 5000 and 4800 rows); the dual GEMV at one row."""
    T = gpu_lib
    say(f"prefill_dual in={i} out={o} k={k} M={M} interleave={il}")
    pa, pb, ya, yb = prefill_dual_case(T, synth.Shape(1, 256, L, k, i, o, il), M, 1300 + M + k)
    assert gate(ya, oracle_y(pa)) <= TOL
    assert gate(yb, oracle_y(pb)) <= TOL


@pytest.mark.parametrize("M", [8, 16, 32])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_prefill_dual_qwen_full(gpu_lib, k, M):
    T = gpu_lib
    say(f"prefill_dual qwen-up k={k} M={M} (whole outputs)")
    pa, pb, ya, yb = prefill_dual_case(T, synth.Shape(1, 256, L, k, QWEN_IN, QWEN_OUT), M,
                                       1320 + k + M)
    assert gate(ya, oracle_y_full(pa)) <= TOL
    assert gate(yb, oracle_y_full(pb)) <= TOL


def test_prefill_dual_too_many_rows_for_one_launch(gpu_lib):
    """More than 144 rows per workgroup on half the compute units: the two
    projections run one launch each."""
    T = gpu_lib
    n = 144 * (T_cus() // 2) + 1
    say(f"prefill_dual in=256 out={n} k=3 M=5")
    pa, pb, ya, yb = prefill_dual_case(T, synth.Shape(1, 256, L, 3, 256, n), 5, 1340)
    assert gate(ya, oracle_y_full(pa)) <= TOL
    assert gate(yb, oracle_y_full(pb)) <= TOL


def T_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# ------------------------------------------------------------ maximum sizes
MAXF = 1 << 19  # largest in/out feature count the library accepts


@pytest.mark.parametrize("k", [2, 4])
def test_gemv_longest_rows(gpu_lib, k):
    """2^19 inputs (2048 blocks per row): the long-row path of the GEMV."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, MAXF, 20)
    p = synth.make_problem(shape, 1, CFG["test"], proj=960 + k)
    say(f"gemv in=2^19 out=20 k={k}")
    y = bf16_to_f64(run(T, Dev(p, T), op="gemv"))
    assert gate(y, oracle_y(p)) <= TOL


def test_gemv_most_rows(gpu_lib):
    """2^19 output rows of 256 inputs, every output checked."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 2, 256, MAXF)
    p = synth.make_problem(shape, 1, CFG["test"], proj=970)
    say("gemv in=256 out=2^19 k=2")
    y = bf16_to_f64(run(T, Dev(p, T), op="gemv"))
    assert gate(y, oracle_y_full(p)) <= TOL


@pytest.mark.parametrize("C", [7936, 8192])
def test_axis0_codes_near_2gib(gpu_lib, C):
    """Axis 0, 2^19 stored rows at k = 4: 7936 columns give 1.94 GiB of codes
    (buffer-addressed loads with lane offsets just below 2^31), 8192 columns
    exactly 2 GiB (the 64-bit pointer path). Checked on sampled columns: the
    whole output would take the oracle 4.3e9 decoded weights."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 4, MAXF, C)
    p = synth.make_problem(shape, 1, CFG["test"], proj=990 + C // 256)
    say(f"scatter in=2^19 out={C} k=4 ({p.codes.nbytes / 2**30:.2f} GiB of codes)")
    y = bf16_to_f64(run(T, Dev(p, T), op="scatter"))
    for a, b in ((0, 16), (C // 2 - 8, C // 2 + 8), (C - 16, C)):
        ref = oracle_y(p, a, b)[:, a:b]
        assert gate(y[:, a:b], ref) <= TOL, (a, b)


@pytest.mark.parametrize("M", [1, 4])
def test_axis0_most_input_rows(gpu_lib, M):
    """Axis 0 with 2^19 stored (input) rows over 256 output columns: 4096 rows
    per split."""
    T = gpu_lib
    shape = synth.Shape(0, 256, L, 3, MAXF, 256)
    p = synth.make_problem(shape, M, CFG["test"], proj=980 + M)
    say(f"axis0 in=2^19 out=256 M={M} k=3")
    d = Dev(p, T)
    y = run(T, d, op="scatter") if M == 1 else run(T, d)
    assert gate(bf16_to_f64(y), oracle_y(p)) <= TOL
