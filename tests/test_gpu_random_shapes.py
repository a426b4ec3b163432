"""GPU parity on seeded random geometries: every compute entry point (GEMV,
dual GEMV, scatter, prefill on both axes, dual prefill) at random k, block
counts, row counts (including 1, 16, 17, 68 and counts that leave ragged row
groups), activation batch sizes and code layouts, against the CPU oracle,
with a second call checked bit-identical to the first; and axis 0 at wide
outputs, where the row split changes plan.

The geometry of case c is drawn from its own generator (seed 20000 + c,
40000 + c for the dual-prefill cases, 50000 + c for the wide axis-0 ones,
60000 + c for the balanced prefill, 70000 + c for the scatter whose bands
meet in one launch), so a failing case is named by its index alone and
reruns unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth
from helpers import TOL, Dev, bf16_bits, bf16_to_f64, gate, say, with_x

pytestmark = pytest.mark.gpu
ROW_CHOICES = [1, 7, 16, 17, 63, 68, 100, 255, 300, 1000, 2049, 4111]


def oracle_y(p):
    s = p.shape
    return oracle.fused_f64(p.x, p.codes, p.scales, p.lut, s.axis, s.T, s.L, s.k,
                            s.in_features, s.out_features, block_interleave=s.block_interleave)


def draw_case(c):
    rng = np.random.default_rng(20000 + c)
    axis = int(rng.integers(0, 2))
    k = int(rng.integers(2, 5))
    nb = int(rng.integers(1, 25))
    rows = int(rng.choice(ROW_CHOICES))
    il = 2 if (nb % 2 == 0 and rng.random() < 0.3) else 0
    i, o = (256 * nb, rows) if axis == 1 else (rows, 256 * nb)
    ops = ["prefill", "gemv", "dual"] if axis == 1 else ["prefill", "scatter"]
    op = str(rng.choice(ops))
    M = 1 if op != "prefill" else int(rng.integers(1, 33))
    return synth.Shape(axis, 256, 12, k, i, o, il), op, M


def call(T, d, op, M):
    x = d.x.reshape(-1) if M == 1 and op != "prefill" else d.x
    if op == "gemv":
        return T.gemv(x, d.codes, d.scales, d.lut, d.shape)
    if op == "scatter":
        return T.gemv_scatter(x, d.codes, d.scales, d.lut, d.shape)
    return T.prefill(x, d.codes, d.scales, d.lut, d.shape)


@pytest.mark.parametrize("c", range(96))
def test_random_geometry(gpu_lib, c):
    run_case(gpu_lib, c, *draw_case(c))


def draw_dual_prefill_case(c):
    rng = np.random.default_rng(40000 + c)
    k = int(rng.integers(2, 5))
    nb = int(rng.integers(1, 25))
    rows = int(rng.choice(ROW_CHOICES))
    il = 2 if (nb % 2 == 0 and rng.random() < 0.3) else 0
    M = int(rng.integers(1, 33))
    return synth.Shape(1, 256, 12, k, 256 * nb, rows, il), "pdual", M


@pytest.mark.parametrize("c", range(32))
def test_random_geometry_dual_prefill(gpu_lib, c):
    run_case(gpu_lib, 1000 + c, *draw_dual_prefill_case(c))


def draw_axis0_case(c):
    """Axis 0 with wide outputs (up to 300 column tiles) and few to many stored
    rows: both split plans (whole bands, and the finer one with a partial
    band, one to eight waves per workgroup), at most 8M weights per case."""
    rng = np.random.default_rng(50000 + c)
    k = int(rng.integers(2, 5))
    nb = int(rng.integers(1, 151))
    cap = max(1, (8 << 20) // (256 * nb))
    rows = int(min(cap, rng.choice([1, 9, 33, 96, 320, 1000, 2050, 4111])))
    il = 2 if (nb % 2 == 0 and rng.random() < 0.3) else 0
    op = str(rng.choice(["scatter", "prefill"]))
    M = 1 if op == "scatter" else int(rng.integers(1, 33))
    return synth.Shape(0, 256, 12, k, rows, 256 * nb, il), op, M


@pytest.mark.parametrize("c", range(32))
def test_random_geometry_axis0_splits(gpu_lib, c):
    run_case(gpu_lib, 2000 + c, *draw_axis0_case(c))


def draw_balanced_case(c):
    """Axis-1 prefill where the balanced plan applies on 256 compute units:
    ceil(N / 16) = 256 f + L groups with L dividing 256 (f whole groups per
    workgroup, the L leftover groups cut into p = 256 / L <= 8 parts of one or
    more blocks), a ragged last group, random k, batch and layout; drawn again
    until wave 0's share holds a part's tasks (the launcher's condition)."""
    rng = np.random.default_rng(60000 + c)
    while True:
        k = int(rng.integers(2, 5))
        f = int(rng.integers(1, 5))
        L = int(rng.choice([32] if f == 1 else [32, 64, 128]))
        p = 256 // L
        nb = int(rng.integers(p, p + 7))
        nq_max, nq_min = -(-nb // p), nb // p
        if (f * nb + nq_min) // 8 >= nq_max:
            break
    N = 16 * (256 * f + L) - int(rng.integers(0, 16))
    # 5 rows or more (fewer take the GEMV-mapped kernel), two M tiles only at k = 3, 4
    M = int(rng.integers(5, 17 if k == 2 else 21))
    M = max(5, min(M, 200_000_000 // (N * nb * 256)))
    il = 2 if (nb % 2 == 0 and rng.random() < 0.3) else 0
    return synth.Shape(1, 256, 12, k, 256 * nb, N, il), "prefill", M


@pytest.mark.parametrize("c", range(16))
def test_random_geometry_balanced_prefill(gpu_lib, c):
    sh, op, M = draw_balanced_case(c)
    if gpu_lib.workspace_bytes(sh, M, gpu_lib.OP_PREFILL) == 0:
        pytest.skip("the balanced plan does not apply with this device's compute-unit count")
    run_case(gpu_lib, 3000 + c, sh, op, M)


def draw_scatter_tagged_case(c):
    """The scatter at 32 to 120 column tiles (whole bands of at most 8 per
    tile, summed in the partial launch through tagged words where the plan
    keeps whole bands), random stored rows, k and layout."""
    rng = np.random.default_rng(70000 + c)
    k = int(rng.integers(2, 5))
    nb = int(rng.integers(16, 61))
    rows = int(rng.choice([33, 96, 300, 1000, 2050, 4111]))
    il = 2 if (nb % 2 == 0 and rng.random() < 0.3) else 0
    return synth.Shape(0, 256, 12, k, rows, 256 * nb, il), "scatter", 1


@pytest.mark.parametrize("c", range(12))
def test_random_geometry_scatter_tagged(gpu_lib, c):
    run_case(gpu_lib, 4000 + c, *draw_scatter_tagged_case(c))


def run_case(gpu_lib, c, sh, op, M):
    T = gpu_lib
    say(f"random case {c}: axis={sh.axis} k={sh.k} in={sh.in_features} "
        f"out={sh.out_features} M={M} il={sh.block_interleave} op={op}")
    p = synth.make_problem(sh, M, synth.CONFIG_IDS["test"], proj=30000 + c)
    d = Dev(p, T)
    if op == "dual":
        pb = with_x(synth.make_problem(sh, 1, synth.CONFIG_IDS["test"], proj=31000 + c), p.x)
        db = Dev(pb, T)
        x = d.x.reshape(-1)
        ya, yb = T.gemv_dual(x, (d.codes, d.scales, d.lut), (db.codes, db.scales, db.lut), sh)
        ra = T.gemv(x, d.codes, d.scales, d.lut, sh)
        rb = T.gemv(x, db.codes, db.scales, db.lut, sh)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(ya), bf16_bits(ra))
        assert np.array_equal(bf16_bits(yb), bf16_bits(rb))
        assert gate(bf16_to_f64(yb.reshape(1, -1)), oracle_y(pb)) <= TOL
        y, again = ya, ra
    elif op == "pdual":
        pb = with_x(synth.make_problem(sh, M, synth.CONFIG_IDS["test"], proj=31000 + c), p.x)
        db = Dev(pb, T)
        ya, yb = T.prefill_dual(d.x, (d.codes, d.scales, d.lut), (db.codes, db.scales, db.lut), sh)
        ya2, yb2 = T.prefill_dual(d.x, (d.codes, d.scales, d.lut), (db.codes, db.scales, db.lut),
                                  sh)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(ya), bf16_bits(ya2))
        assert np.array_equal(bf16_bits(yb), bf16_bits(yb2))
        assert gate(bf16_to_f64(yb.reshape(M, -1)), oracle_y(pb)) <= TOL
        y = ya
    else:
        y = call(T, d, op, M)
        again = call(T, d, op, M)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), bf16_bits(again))
    assert gate(bf16_to_f64(y.reshape(M, -1)), oracle_y(p)) <= TOL
