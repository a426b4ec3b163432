"""GPU parity of the balanced axis-1 prefill plan: whole 16-row groups per
workgroup, the leftover groups cut by blocks into parts that meet through the
workspace (the last part to arrive sums them). Against the oracle, against the
plan without a workspace, bit-exact where the sums are exact, with a workspace
of arbitrary contents, and replayed from a captured graph.

The plan applies where the 16-row groups outnumber the workgroups (one per
compute unit) by a remainder that divides them (not at k = 2 with more than
16 rows); each test names a shape where it applies on a 256-CU device and
skips where workspace_bytes says it does not.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import TOL, Dev, bf16_bits, bf16_to_f64, gate, oracle_y_full, say

pytestmark = pytest.mark.gpu
CFG = synth.CONFIG_IDS
L = 12


def oracle_y(p):
    s = p.shape
    return oracle.fused_f64(p.x, p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k,
                            s.in_features, s.out_features, 0, None,
                            block_interleave=s.block_interleave)


def split_bytes(T, shape, M):
    n = T.workspace_bytes(shape, M, T.OP_PREFILL)
    if n == 0:
        pytest.skip(f"the balanced plan does not apply to {shape} at M={M} on this device")
    return n


def prefill(T, d, ws=None, balanced=True):
    y = T.prefill(d.x, d.codes, d.scales, d.lut, d.shape, workspace=ws, balanced=balanced)
    torch.cuda.synchronize()
    return y


# (in, out, k, M, block interleave): leftover groups cut into 4 (17408 rows:
# 1088 groups = 4 x 256 + 64) or 8 (16896 and 8704 rows) parts; one
# or two blocks per part (1536 inputs: 6 blocks in parts of 1, 2, 1, 2); a
# last group of 8 rows (17400); one full group per workgroup (4608 rows).
SHAPES = [(1024, 17408, 2, 5, 0),
          (1536, 17408, 3, 16, 0),
          (1024, 17400, 4, 32, 0),
          (2048, 16896, 3, 20, 2),
          (2048, 4608, 3, 9, 0),
          (4096, 8704, 4, 17, 0),
          (5120, 17408, 3, 24, 2)]


@pytest.mark.parametrize("i,o,k,M,il", SHAPES)
def test_split_prefill_against_oracle(gpu_lib, i, o, k, M, il):
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o, il)
    split_bytes(T, shape, M)
    p = synth.make_problem(shape, M, CFG["test"], proj=2100 + k + M)
    say(f"split prefill in={i} out={o} k={k} M={M} interleave={il}")
    d = Dev(p, T)
    y = bf16_to_f64(prefill(T, d))
    ref = oracle_y_full(p)
    assert gate(y, ref) <= TOL
    # the plan without a workspace: the same sums in another order
    y0 = bf16_to_f64(prefill(T, d, balanced=False))
    assert gate(y0, ref) <= TOL


@pytest.mark.parametrize("i,o,k,M", [(1536, 17408, 3, 32), (1024, 17400, 2, 8), (2048, 4608, 4, 16),
                                     (5120, 17408, 4, 32), (5120, 17408, 2, 16)])
def test_split_integer_codebook_bit_exact(gpu_lib, i, o, k, M):
    """Integer codebook, activations and power-of-two scales: every partial and
    every sum of parts is exact in float32, so each output is the unique bf16
    of the exact sum, on the leftover rows as on the others."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, k, i, o)
    split_bytes(T, shape, M)
    g = np.random.default_rng(2200 + M + k)
    p0 = synth.make_problem(shape, M, CFG["test"], proj=2200 + M)
    xi = g.integers(-3, 4, (M, i)).astype(np.float32)
    p = synth.Problem(shape, M, p0.codes, synth.integer_lut(),
                      g.choice(np.array([0.5, 1.0, 2.0], np.float32), shape.rows),
                      synth.to_bf16_bits(xi))
    say(f"split prefill integer codebook in={i} out={o} k={k} M={M}")
    y = bf16_bits(prefill(T, Dev(p, T)))
    exact = oracle_y(p)
    assert np.all(np.abs(exact) < 2**24)
    assert np.array_equal(y, synth.to_bf16_bits(exact.astype(np.float32)))


def test_split_workspace_any_contents(gpu_lib):
    """The workspace needs no clearing: from random bits, shared with another
    geometry (other part counts), and holding the parts of a call on other
    activations, every call gives the bits of a fresh one; a part of another
    call is never added."""
    T = gpu_lib
    sa = synth.Shape(1, 256, L, 2, 1024, 17408)
    sb = synth.Shape(1, 256, L, 3, 2048, 16896)
    na, nb_ = split_bytes(T, sa, 16), split_bytes(T, sb, 16)
    pa = synth.make_problem(sa, 16, CFG["test"], proj=2300)
    pb = synth.make_problem(sb, 16, CFG["test"], proj=2301)
    pa2 = synth.make_problem(sa, 16, CFG["test"], proj=2303)  # other activations, same codes shape
    da, db, da2 = Dev(pa, T), Dev(pb, T), Dev(pa2, T)
    n = max(na, nb_) // 4
    g = torch.Generator().manual_seed(2302)
    ws = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, generator=g).cuda().view(torch.float32)
    say("split prefill, workspace of random bits, then shared by two geometries")
    ta = prefill(T, da, ws)
    ya = bf16_bits(ta)
    assert gate(bf16_to_f64(ta), oracle_y_full(pa)) <= TOL
    tb = prefill(T, db, ws)
    yb = bf16_bits(tb)
    assert gate(bf16_to_f64(tb), oracle_y_full(pb)) <= TOL
    ya2 = bf16_bits(prefill(T, da2, ws))
    assert np.array_equal(ya2, bf16_bits(prefill(T, da2, torch.empty_like(ws))))
    for _ in range(3):
        assert np.array_equal(bf16_bits(prefill(T, da, ws)), ya)
        assert np.array_equal(bf16_bits(prefill(T, da2, ws)), ya2)
        assert np.array_equal(bf16_bits(prefill(T, db, ws)), yb)


def test_split_not_captured(gpu_lib):
    """A captured call takes the plan without the split (a replay would reuse
    the call's tag): every replay, with eager balanced calls on the same
    workspace in between, equals the eager unbalanced result bit for bit,
    and the eager calls keep their own bits."""
    T = gpu_lib
    shape = synth.Shape(1, 256, L, 4, 1024, 17408)
    nbytes = split_bytes(T, shape, 32)
    p = synth.make_problem(shape, 32, CFG["test"], proj=2400)
    d = Dev(p, T)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty((32, 17408), dtype=torch.bfloat16, device="cuda")
    say("split prefill under stream capture, replayed three times")
    plain = bf16_bits(prefill(T, d, balanced=False))
    T.prefill(d.x, d.codes, d.scales, d.lut, d.shape, workspace=ws, y=y)
    torch.cuda.synchronize()
    balanced = bf16_bits(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        T.prefill(d.x, d.codes, d.scales, d.lut, d.shape, workspace=ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        T.prefill(d.x, d.codes, d.scales, d.lut, d.shape, workspace=ws, y=y)
    for r in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), plain), r
        T.prefill(d.x, d.codes, d.scales, d.lut, d.shape, workspace=ws, y=y)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), balanced), r


# ------------------------------------------------ the scatter's in-launch sum
FUSED = synth.Shape(0, 256, L, 3, 1000, 5120)  # 40 tiles x 6 bands of whole-band workgroups


@pytest.mark.parametrize("fill", [None, 0x00, 0xFF, 0x7FC00000])
def test_scatter_tagged_sum_any_contents(gpu_lib, fill):
    """The scatter whose bands meet through tagged words (whole bands, few
    per tile): a fresh workspace, one of zero bytes, of all-ones bytes, or of
    quiet NaNs gives the same bits, within tolerance of the oracle, on three
    calls in a row."""
    T = gpu_lib
    n = T.workspace_bytes(FUSED, 1, T.OP_GEMV_SCATTER)
    assert n == 240 * 128 * 8, n  # the tagged-word plan
    p = synth.make_problem(FUSED, 1, CFG["test"], proj=2500)
    d = Dev(p, T)
    say(f"scatter tagged sum, workspace fill {fill}")
    ref = bf16_bits(T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, FUSED,
                                   workspace=torch.empty(n // 4, dtype=torch.float32, device="cuda")))
    if fill is None:
        ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    elif fill == 0x7FC00000:
        ws = torch.full((n // 4,), fill, dtype=torch.int32, device="cuda").view(torch.float32)
    else:
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda").view(torch.float32)
    for _ in range(3):
        y = T.gemv_scatter(d.x.reshape(-1), d.codes, d.scales, d.lut, FUSED, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), ref)
    assert gate(bf16_to_f64(y.reshape(1, -1)), oracle_y(p)) <= TOL


def test_scatter_tagged_sum_under_capture(gpu_lib):
    """Under stream capture the scatter takes float32 partials and a reduce
    launch summing the bands in the same order: every replay, with eager
    calls on the same workspace in between, equals the eager bits."""
    T = gpu_lib
    n = T.workspace_bytes(FUSED, 1, T.OP_GEMV_SCATTER)
    p = synth.make_problem(FUSED, 1, CFG["test"], proj=2501)
    d = Dev(p, T)
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    y = torch.empty(5120, dtype=torch.bfloat16, device="cuda")
    xv = d.x.reshape(-1)
    say("scatter tagged sum under stream capture")
    T.gemv_scatter(xv, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    torch.cuda.synchronize()
    eager = bf16_bits(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        T.gemv_scatter(xv, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        T.gemv_scatter(xv, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    for r in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), eager), r
        T.gemv_scatter(xv, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), eager), r


@pytest.mark.parametrize("M", [2, 5, 8])
def test_axis0_prefill_tagged_sum(gpu_lib, M):
    """The axis-0 prefill at M <= 8 sums its bands in the partial launch too:
    against the oracle, on a workspace of all-ones bytes, bit-identical over
    three calls and to a call under stream capture (float partials, then the
    reduce launch in the same band order)."""
    T = gpu_lib
    n = T.workspace_bytes(FUSED, M, T.OP_PREFILL)
    assert n == 240 * M * 128 * 8, n  # tagged words
    p = synth.make_problem(FUSED, M, CFG["test"], proj=2600 + M)
    d = Dev(p, T)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda").view(torch.float32)
    y = torch.empty((M, 5120), dtype=torch.bfloat16, device="cuda")
    say(f"axis-0 prefill tagged sum M={M}")
    T.prefill(d.x, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    torch.cuda.synchronize()
    first = bf16_bits(y)
    assert gate(bf16_to_f64(y), oracle_y(p)) <= TOL
    for _ in range(2):
        T.prefill(d.x, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), first)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        T.prefill(d.x, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        T.prefill(d.x, d.codes, d.scales, d.lut, FUSED, workspace=ws, y=y)
    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), first)
