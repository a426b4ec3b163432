"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- a closed form, an invariant of the bitshift trellis,
brute force on tiny inputs, or a library routine (numpy, torch, Python big
integers). Together they are chosen so that a plausible slip anywhere in the
oracle (window direction, wrap, bit order, rounding placement, scale index,
transposed contraction, dropped term) fails at least one of them.

Pages: the diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0, page 60
(tiled-prefill.ts weight-tile decode; vector-expand.ts) and page 59
(scatter.ts row loop; splitk-prefill.ts).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from dequant_gemm_trellis_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L = 12


# ----------------------------------------------------------------- helpers
def bigint(block):
    """The block's bitstring as a Python integer (word j at bits 32j..)."""
    v = 0
    for j, w in enumerate(np.asarray(block, dtype=np.uint64).tolist()):
        v |= int(w) << (32 * j)
    return v


def rot_windows(block, T, k, L=L):
    """Closed form: window t = low L bits of the T*k-bit string rotated right
    by (T-1-t)*k (a cyclic rotation is exactly the tail-biting wrap)."""
    n = T * k
    B = bigint(block)
    mask = (1 << n) - 1
    out = []
    for t in range(T):
        p = (T - 1 - t) * k
        rot = ((B >> p) | (B << (n - p))) & mask if p else B
        out.append(rot & ((1 << L) - 1))
    return np.array(out, dtype=np.uint32)


def torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def brute_expand(codes, scales, lut, T, k):
    """Independent expand: big-integer windows, numpy float32 product,
    torch's bf16 cast."""
    rows, wpr = codes.shape
    wpb = T * k // 32
    nb = wpr // wpb
    W = np.empty((rows, nb * T), dtype=np.uint16)
    for r in range(rows):
        for b in range(nb):
            win = rot_windows(codes[r, b * wpb:(b + 1) * wpb], T, k)
            prod = lut[win].astype(np.float32) * np.float32(scales[r])
            W[r, b * T:(b + 1) * T] = torch_bf16_bits(prod)
    return W


def f64(bits):
    return oracle.bf16_bits_to_f64(bits)


# ------------------------------------------------------------ bf16 rounding
def test_bf16_rne_matches_torch_random():
    g = np.random.default_rng(1)
    a = np.concatenate([
        g.standard_normal(400_000).astype(np.float32),
        (g.standard_normal(300_000) * 1e30).astype(np.float32),
        (g.standard_normal(300_000) * 1e-30).astype(np.float32),
        g.integers(0, 2**32, 200_000, dtype=np.uint32).view(np.float32),
    ])
    a = a[np.isfinite(a)]
    # values that would round to infinity are outside the method's range
    a = a[np.abs(a) < 3.0e38]
    assert np.array_equal(oracle.bf16_rne_array(a), torch_bf16_bits(a))


def test_bf16_rne_ties_go_to_even():
    hi = np.arange(0, 0x7F80, 7, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    out = oracle.bf16_rne_array(ties)
    # a tie rounds to the even neighbour: up iff the kept half is odd
    expect = np.where(hi & 1, hi + 1, hi).astype(np.uint16)
    assert np.array_equal(out, expect)
    assert np.array_equal(out, torch_bf16_bits(ties))


def test_weight_is_f32_product_then_bf16():
    g = np.random.default_rng(2)
    v = g.standard_normal(2_000_000).astype(np.float32)
    s = g.uniform(0.5, 1.5, 2_000_000).astype(np.float32)
    p32 = v * s  # one IEEE float32 multiply
    # pairs where rounding the exact product straight to bf16 differs from
    # rounding the float32 product: float32 lands exactly on a bf16 tie
    exact = v.astype(np.float64) * s.astype(np.float64)  # exact in float64
    on_tie = (p32.view(np.uint32) & 0xFFFF) == 0x8000
    idx = np.nonzero(on_tie & (exact != p32.astype(np.float64)))[0]
    assert idx.size > 0, "the sample must contain double-rounding cases"
    sample = np.concatenate([idx, np.arange(5000)])
    got = np.array([oracle.weight(float(v[i]), float(s[i])) for i in sample], dtype=np.uint16)
    assert np.array_equal(got, torch_bf16_bits(p32[sample]))
    # and at least one of them differs from rounding the exact product once,
    # straight to the bf16 grid (8 significant bits, ties to even)
    def bf16_single(x):
        import math
        m, e = math.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
        q = m * 256.0          # 8 significant bits
        r = round(q)           # Python round: ties to even, exact on floats
        return torch_bf16_bits(np.array([math.ldexp(r / 256.0, e)], dtype=np.float32))[0]
    singles = np.array([bf16_single(float(exact[i])) for i in idx], dtype=np.uint16)
    assert np.any(singles != got[: idx.size])


# ------------------------------------------------------------------ windows
@pytest.mark.parametrize("T,k", [(16, 2), (8, 4)])
def test_single_word_block_is_32bit_rotation(T, k):
    g = np.random.default_rng(3)
    for w in g.integers(0, 2**32, 200, dtype=np.uint32):
        w = int(w)
        got = oracle.windows(np.array([w], dtype=np.uint32), T, k, L)
        for t in range(T):
            p = (T - 1 - t) * k
            rot = ((w >> p) | (w << (32 - p))) & 0xFFFFFFFF if p else w
            assert got[t] == rot & 0xFFF


@pytest.mark.parametrize("T,k", [(32, 3), (256, 2), (256, 3), (256, 4), (64, 2)])
def test_windows_match_bigint_rotation(T, k):
    g = np.random.default_rng(4 + k)
    for _ in range(6):
        block = g.integers(0, 2**32, T * k // 32, dtype=np.uint32)
        want = rot_windows(block, T, k)
        assert np.array_equal(oracle.windows(block, T, k, L), want)
        assert np.array_equal(oracle.windows_from_bits(block, T, k, L), want)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_trellis_shift_invariant(k):
    """Consecutive weights are neighbouring states of a bitshift trellis: the
    low L-k bits of window t equal window t+1 shifted down by k (cyclically,
    t = T-1 is followed by t = 0)."""
    T = 256
    g = np.random.default_rng(10 + k)
    for _ in range(8):
        block = g.integers(0, 2**32, T * k // 32, dtype=np.uint32)
        w = oracle.windows(block, T, k, L)
        for t in range(T):
            assert w[t] & ((1 << (L - k)) - 1) == w[(t + 1) % T] >> k


@pytest.mark.parametrize("k", [2, 3, 4])
def test_symbols_tile_the_block_exactly(k):
    """Bit budget: the k low bits of the T windows, placed at (T-1-t)*k,
    rebuild the T*k-bit block exactly -- nothing missing, nothing shared."""
    T = 256
    g = np.random.default_rng(20 + k)
    for _ in range(8):
        block = g.integers(0, 2**32, T * k // 32, dtype=np.uint32)
        w = oracle.windows(block, T, k, L)
        rebuilt = 0
        for t in range(T):
            rebuilt |= int(w[t] & ((1 << k) - 1)) << ((T - 1 - t) * k)
        assert rebuilt == bigint(block)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_single_bit_lies_in_exactly_L_over_k_windows(k):
    T = 256
    n = T * k
    nwords = n // 32
    g = np.random.default_rng(30 + k)
    for q in list(range(0, 40)) + list(range(n - 40, n)) + list(g.integers(0, n, 30)):
        q = int(q)
        block = np.zeros(nwords, dtype=np.uint32)
        block[q // 32] = np.uint32(1 << (q % 32))
        w = oracle.windows(block, T, k, L)
        nz = np.nonzero(w)[0]
        assert nz.size == L // k
        for t in nz:
            p = (T - 1 - int(t)) * k
            assert w[t] == 1 << ((q - p) % n)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_bit_flip_changes_only_its_own_block(k):
    T = 256
    g = np.random.default_rng(40 + k)
    shape = synth.Shape(1, T, L, k, 3 * T, 2)
    codes = g.integers(0, 2**32, (2, shape.words_per_row), dtype=np.uint32)
    # 4096 distinct bf16-representable entries, so W reveals the windows
    lut = ((np.arange(1 << L, dtype=np.uint32) + 0x3F80) << 16).view(np.float32)
    scales = np.ones(2, dtype=np.float32)
    base = oracle.expand(codes, scales, lut, 1, T, L, k, 3 * T, 2)
    for _ in range(20):
        r = int(g.integers(0, 2))
        bit = int(g.integers(0, shape.words_per_row * 32))
        c2 = codes.copy()
        c2[r, bit // 32] ^= np.uint32(1 << (bit % 32))
        W2 = oracle.expand(c2, scales, lut, 1, T, L, k, 3 * T, 2)
        changed = np.argwhere(base != W2)
        assert len(changed) == L // k
        blk = bit // (T * k)
        assert np.all(changed[:, 0] == r)
        assert np.all(changed[:, 1] // T == blk)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_constant_patterns(k):
    T = 256
    nw = T * k // 32
    assert np.all(oracle.windows(np.zeros(nw, np.uint32), T, k, L) == 0)
    assert np.all(oracle.windows(np.full(nw, 0xFFFFFFFF, np.uint32), T, k, L) == 0xFFF)


def test_periodic_patterns():
    T = 256
    # k=2, every even bit set: each window starts on an even bit -> 0x555
    assert np.all(oracle.windows(np.full(16, 0x55555555, np.uint32), T, 2, L) == 0x555)
    # k=4, nibbles 0..7 repeating: window t starts at nibble j=(T-1-t) mod 8
    w = oracle.windows(np.full(32, 0x76543210, np.uint32), T, 4, L)
    for t in range(T):
        j = (T - 1 - t) % 8
        assert w[t] == j | (((j + 1) % 8) << 4) | (((j + 2) % 8) << 8)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_wraparound_closed_form(k):
    """Window 0 takes the top k bits of the block followed by its low L-k
    bits; window T-1 is the block's low L bits."""
    T = 256
    n = T * k
    g = np.random.default_rng(50 + k)
    block = g.integers(0, 2**32, n // 32, dtype=np.uint32)
    B = bigint(block)
    w = oracle.windows(block, T, k, L)
    assert w[0] == (B >> (n - k)) | ((B & ((1 << (L - k)) - 1)) << k)
    assert w[T - 1] == B & 0xFFF


def test_golden_windows():
    """Hand-derived windows (tests/golden/windows_hand.txt)."""
    path = os.path.join(GOLDEN, "windows_hand.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        T, k, words, t, want = line.split()
        block = np.array([int(w, 16) for w in words.split(",")], dtype=np.uint32)
        got = oracle.windows(block, int(T), int(k), L)[int(t)]
        assert got == int(want, 16), line
        n += 1
    assert n >= 8


# ------------------------------------------------------------------- expand
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_expand_matches_brute_force(axis, k):
    T = 256
    shape = synth.Shape(axis, T, L, k, 512 if axis == 1 else 5, 5 if axis == 1 else 512)
    p = synth.make_problem(shape, 1, synth.CONFIG_IDS["test"], proj=k)
    W = oracle.expand(p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                      shape.out_features)
    assert W.shape == (shape.rows, shape.cols)
    assert np.array_equal(W, brute_expand(p.codes, p.scales, p.lut, T, k))


def test_expand_uses_the_stored_row_scale():
    """Axis 0: scales index the stored row (the input feature)."""
    T, k = 256, 3
    shape = synth.Shape(0, T, L, k, 4, 256)
    codes = np.zeros((4, shape.words_per_row), dtype=np.uint32)  # every window 0
    lut = np.zeros(1 << L, dtype=np.float32)
    lut[0] = 1.0
    scales = np.array([0.5, 1.0, 2.0, 4.0], dtype=np.float32)
    W = oracle.expand(codes, scales, lut, 0, T, L, k, 4, 256)
    assert np.array_equal(f64(W), np.repeat(scales[:, None], 256, axis=1).astype(np.float64))


# --------------------------------------------------------------- contraction
@pytest.mark.parametrize("axis", [0, 1])
def test_matmul_matches_numpy_within_bound(axis):
    T, k = 256, 2
    shape = synth.Shape(axis, T, L, k, 768 if axis == 1 else 300, 300 if axis == 1 else 768)
    p = synth.make_problem(shape, 3, synth.CONFIG_IDS["test"], proj=7)
    W = oracle.expand(p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                      shape.out_features)
    y = oracle.matmul_f64(p.x, W, axis, shape.in_features, shape.out_features)
    X, Wd = f64(p.x), f64(W)
    Wnk = Wd if axis == 1 else Wd.T          # [out, in]
    ref = X @ Wnk.T
    bound = 2 * shape.in_features * 2.0**-53 * (np.abs(X) @ np.abs(Wnk).T)
    assert np.all(np.abs(y - ref) <= bound)


@pytest.mark.parametrize("axis", [0, 1])
def test_one_hot_x_returns_stored_weights_exactly(axis):
    T, k = 256, 3
    shape = synth.Shape(axis, T, L, k, 512 if axis == 1 else 40, 40 if axis == 1 else 512)
    p = synth.make_problem(shape, 1, synth.CONFIG_IDS["test"], proj=11)
    W = oracle.expand(p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                      shape.out_features)
    n_in = shape.in_features
    cols = sorted({0, 1, min(255, n_in - 2), min(256, n_in - 1) // 2, n_in - 1})
    x = synth.one_hot_x(len(cols), shape.in_features, cols)
    y = oracle.fused_f64(x, p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                         shape.out_features)
    for m, j in enumerate(cols):
        want = W[:, j] if axis == 1 else W[j, :]
        assert np.array_equal(y[m], f64(want))


@pytest.mark.parametrize("axis", [0, 1])
def test_integer_codebook_is_exact(axis):
    T, k = 256, 4
    shape = synth.Shape(axis, T, L, k, 1024 if axis == 1 else 64, 64 if axis == 1 else 1024)
    g = np.random.default_rng(60 + axis)
    codes = synth.codes(shape, synth.CONFIG_IDS["test"], 1, 13)
    lut = synth.integer_lut(L)
    scales = g.choice(np.array([0.5, 1.0, 2.0], dtype=np.float32), shape.rows)
    xi = g.integers(-4, 5, (2, shape.in_features))
    x = synth.to_bf16_bits(xi.astype(np.float32))
    y = oracle.fused_f64(x, codes, scales, lut, axis, T, L, k, shape.in_features,
                         shape.out_features)
    # integer reference: window -> (w mod 15) - 7 via the closed-form windows
    Wint = np.empty((shape.rows, shape.cols), dtype=np.float64)
    wpb = T * k // 32
    for r in range(shape.rows):
        for b in range(shape.cols // T):
            win = rot_windows(codes[r, b * wpb:(b + 1) * wpb], T, k)
            Wint[r, b * T:(b + 1) * T] = ((win % 15).astype(np.int64) - 7) * float(scales[r])
    Wnk = Wint if axis == 1 else Wint.T
    assert np.array_equal(y, xi.astype(np.float64) @ Wnk.T)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("M", [1, 3])
def test_fused_equals_expand_then_matmul_bitwise(axis, M):
    T, k = 256, 3
    shape = synth.Shape(axis, T, L, k, 512 if axis == 1 else 96, 96 if axis == 1 else 512)
    p = synth.make_problem(shape, M, synth.CONFIG_IDS["test"], proj=17)
    W = oracle.expand(p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                      shape.out_features)
    y1 = oracle.matmul_f64(p.x, W, axis, shape.in_features, shape.out_features)
    y2 = oracle.fused_f64(p.x, p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                          shape.out_features)
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))
    y3 = oracle.fused_f64(p.x, p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                          shape.out_features, 7, 40)
    assert np.array_equal(y3[:, 7:40], y1[:, 7:40])
    assert not np.any(y3[:, :7]) and not np.any(y3[:, 40:])


# ------------------------------------------------------ block interleave 2
def test_interleave_layout_brute_force():
    """Block interleave 2 ([P60] vector-expand.ts, [P59] scatter.ts when
    INTERLEAVE is set): block pairs outermost, then stored rows, then the
    pair's two blocks, then the words of a block. Words are labelled with
    their (row, block, word) and the rewritten array is compared with that
    order written out as nested loops."""
    rows, nb, wpb = 3, 4, 2
    label = lambda r, b, w: 1000 * r + 10 * b + w
    codes = np.array([label(r, b, w) for r in range(rows) for b in range(nb) for w in range(wpb)],
                     dtype=np.uint32)
    expect = []
    for pair in range(nb // 2):
        for r in range(rows):
            for half in range(2):
                for w in range(wpb):
                    expect.append(label(r, 2 * pair + half, w))
    il = oracle.interleave_blocks(codes, rows, nb, wpb)
    assert il.tolist() == expect
    assert np.array_equal(oracle.deinterleave_blocks(il, rows, nb, wpb), codes)
    with pytest.raises(ValueError):
        oracle.interleave_blocks(codes[: rows * 3 * wpb], rows, 3, wpb)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("k", [2, 3, 4])
def test_expand_reads_the_interleaved_layout(axis, k):
    """The oracle's block addressing under interleave 2 (its offset formula)
    against the layout produced by a reshape and transpose: the decoded
    matrix must not depend on the layout."""
    T = 256
    rows, cols = 5, 4 * T
    shape = synth.Shape(axis, T, L, k, cols if axis == 1 else rows, rows if axis == 1 else cols)
    p = synth.make_problem(shape, 1, synth.CONFIG_IDS["test"], proj=23)
    W0 = oracle.expand(p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                       shape.out_features)
    c2 = oracle.interleave_blocks(p.codes, rows, cols // T, T * k // 32)
    assert not np.array_equal(c2, p.codes.ravel())
    W2 = oracle.expand(c2, p.scales, p.lut, axis, T, L, k, shape.in_features,
                       shape.out_features, block_interleave=2)
    assert np.array_equal(W0, W2)
    # brute force on the rewritten array: each block decoded through the
    # closed-form windows at the position the nested-loop order puts it
    wpb = T * k // 32
    for r in range(rows):
        for b in range(cols // T):
            off = ((b // 2) * rows * 2 + r * 2 + b % 2) * wpb
            win = rot_windows(c2[off:off + wpb], T, k)
            vals = np.array([oracle.weight(float(p.lut[w]), float(p.scales[r])) for w in win],
                            dtype=np.uint16)
            assert np.array_equal(W2[r, b * T:(b + 1) * T], vals)


@pytest.mark.parametrize("axis", [0, 1])
def test_fused_reads_the_interleaved_layout(axis):
    T, k, M = 256, 3, 2
    rows, cols = 6, 2 * T
    shape = synth.Shape(axis, T, L, k, cols if axis == 1 else rows, rows if axis == 1 else cols)
    p = synth.make_problem(shape, M, synth.CONFIG_IDS["test"], proj=29)
    y0 = oracle.fused_f64(p.x, p.codes, p.scales, p.lut, axis, T, L, k, shape.in_features,
                          shape.out_features)
    c2 = oracle.interleave_blocks(p.codes, rows, cols // T, T * k // 32)
    y2 = oracle.fused_f64(p.x, c2, p.scales, p.lut, axis, T, L, k, shape.in_features,
                          shape.out_features, block_interleave=2)
    assert np.array_equal(y0.view(np.uint64), y2.view(np.uint64))


def test_interleave_needs_an_even_block_count():
    T, k = 256, 2
    codes = np.zeros(2 * 3 * T * k // 32, dtype=np.uint32)
    scales = np.ones(2, dtype=np.float32)
    lut = np.zeros(4096, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.expand(codes, scales, lut, 1, T, L, k, 3 * T, 2, block_interleave=2)
    with pytest.raises(ValueError):
        oracle.expand(codes, scales, lut, 1, T, L, k, 3 * T, 2, block_interleave=1)
    oracle.expand(codes, scales, lut, 1, T, L, k, 3 * T, 2, block_interleave=0)


# ------------------------------------------------------------ SwiGLU epilogue
def test_silu_closed_forms():
    """silu(0) = 0; sigmoid(ln 3) = 3/4, so silu(ln 3) = (3/4) ln 3 (this also
    fails v * sigmoid(-v), which agrees with silu on the odd identity below);
    silu(v) -> v far right, -> 0 far left."""
    import math

    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert oracle.silu(-math.log(3.0)) == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert oracle.silu(-800.0) == 0.0


def test_silu_odd_part_is_identity():
    """silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1)."""
    rng = np.random.default_rng(7)
    for v in rng.standard_normal(2000) * 6:
        assert oracle.silu(v) - oracle.silu(-v) == pytest.approx(v, rel=1e-13, abs=1e-15)


def test_silu_matches_torch():
    """Against torch's CPU silu in float64 (a library routine)."""
    rng = np.random.default_rng(8)
    v = rng.standard_normal(100_000) * 20
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    got = np.array([oracle.silu(float(a)) for a in v[:5000]])
    np.testing.assert_allclose(got, ref[:5000], rtol=1e-14, atol=1e-300)
    h = oracle.swiglu_f64(v, np.ones_like(v))
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=1e-300)


def test_swiglu_applies_silu_to_the_gate():
    """h = silu(g) * u, not silu(u) * g: g = ln 3, u = 4 gives 3 ln 3; a zero
    gate gives zero whatever u is; the up operand enters linearly."""
    import math

    g = np.array([math.log(3.0), 0.0, math.log(3.0)])
    u = np.array([4.0, 123.0, -8.0])
    h = oracle.swiglu_f64(g, u)
    assert h[0] == pytest.approx(3.0 * math.log(3.0), rel=1e-15)
    assert h[1] == 0.0
    assert h[2] == pytest.approx(-6.0 * math.log(3.0), rel=1e-15)
    with pytest.raises(ValueError):
        oracle.swiglu_f64(np.zeros(3), np.zeros(4))


def test_mlp_up_swiglu_on_one_hot_rows_uses_the_stored_weights():
    """One-hot activation rows select one stored column of each projection
    exactly, so h[m][n] = silu(Wg[n][j_m]) * Wu[n][j_m] with both weights read
    from the oracle's expand (pinned above by brute force)."""
    T, k, i, o = 256, 3, 512, 40
    sh = synth.Shape(1, T, L, k, i, o)
    pg = synth.make_problem(sh, 1, synth.CONFIG_IDS["test"], proj=900)
    pu = synth.make_problem(sh, 1, synth.CONFIG_IDS["test"], proj=901)
    cols = [0, 255, 256, 511]
    x = synth.one_hot_x(len(cols), i, cols)
    h = oracle.mlp_up_swiglu_f64(x, (pg.codes, pg.scales, pg.lut), (pu.codes, pu.scales, pu.lut),
                                 T, L, k, i, o)
    Wg = oracle.bf16_bits_to_f64(oracle.expand(pg.codes, pg.scales, pg.lut, 1, T, L, k, i, o))
    Wu = oracle.bf16_bits_to_f64(oracle.expand(pu.codes, pu.scales, pu.lut, 1, T, L, k, i, o))
    for m, j in enumerate(cols):
        want = torch.nn.functional.silu(torch.from_numpy(Wg[:, j])).numpy() * Wu[:, j]
        np.testing.assert_allclose(h[m], want, rtol=1e-14, atol=0)
