"""CPU oracle for the trellis dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg may import it; the product path never does. The arithmetic
lives in ``trellis_oracle.c`` (plain single-threaded C built with gcc); this
module only marshals numpy arrays into it.

Pinned by ``tests/test_oracle_pins.py`` (closed forms, invariants, brute force,
library routines); no function here is parity-unpinned.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from .build import ensure_built

_lib = C.CDLL(ensure_built())

_u16p = C.POINTER(C.c_uint16)
_u32p = C.POINTER(C.c_uint32)
_u8p = C.POINTER(C.c_uint8)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)

_lib.oracle_bf16_rne.restype = C.c_uint16
_lib.oracle_bf16_rne.argtypes = [C.c_float]
_lib.oracle_bf16_rne_n.restype = None
_lib.oracle_bf16_rne_n.argtypes = [_f32p, C.c_long, _u16p]
_lib.oracle_bf16_to_f64.restype = C.c_double
_lib.oracle_bf16_to_f64.argtypes = [C.c_uint16]
_lib.oracle_block_bits.restype = None
_lib.oracle_block_bits.argtypes = [_u32p, C.c_int, C.c_int, _u8p]
_lib.oracle_window.restype = C.c_uint32
_lib.oracle_window.argtypes = [_u32p, C.c_int, C.c_int, C.c_int, C.c_int]
_lib.oracle_window_from_bits.restype = C.c_uint32
_lib.oracle_window_from_bits.argtypes = [_u8p, C.c_int, C.c_int, C.c_int, C.c_int]
_lib.oracle_weight.restype = C.c_uint16
_lib.oracle_weight.argtypes = [C.c_float, C.c_float]
_lib.oracle_expand.restype = C.c_int
_lib.oracle_expand.argtypes = [_u32p, _f32p, _f32p, C.c_int, C.c_int, C.c_int, C.c_int,
                               C.c_int, C.c_int, C.c_int, _u16p]
_lib.oracle_matmul_f64.restype = C.c_int
_lib.oracle_matmul_f64.argtypes = [_u16p, C.c_int, _u16p, C.c_int, C.c_int, C.c_int, _f64p]
_lib.oracle_fused_f64.restype = C.c_int
_lib.oracle_fused_f64.argtypes = [_u16p, C.c_int, _u32p, _f32p, _f32p, C.c_int, C.c_int,
                                  C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                  C.c_int, _f64p]
_lib.oracle_silu.restype = C.c_double
_lib.oracle_silu.argtypes = [C.c_double]
_lib.oracle_swiglu_f64.restype = None
_lib.oracle_swiglu_f64.argtypes = [_f64p, _f64p, C.c_long, _f64p]


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _dims(axis: int, in_features: int, out_features: int) -> tuple[int, int]:
    return (out_features, in_features) if axis == 1 else (in_features, out_features)


def bf16_rne(f: float) -> int:
    return int(_lib.oracle_bf16_rne(f))


def bf16_rne_array(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    out = np.empty(a.size, dtype=np.uint16)
    _lib.oracle_bf16_rne_n(_p(a, _f32p), a.size, _p(out, _u16p))
    return out


def weight(value: float, scale: float) -> int:
    return int(_lib.oracle_weight(value, scale))


def block_bits(block: np.ndarray, T: int, k: int) -> np.ndarray:
    block = np.ascontiguousarray(block, dtype=np.uint32)
    bits = np.zeros(T * k, dtype=np.uint8)
    _lib.oracle_block_bits(_p(block, _u32p), T, k, _p(bits, _u8p))
    return bits


def windows(block: np.ndarray, T: int, k: int, L: int) -> np.ndarray:
    """All T windows of one block, read directly from the words."""
    block = np.ascontiguousarray(block, dtype=np.uint32)
    return np.array([_lib.oracle_window(_p(block, _u32p), T, k, L, t) for t in range(T)],
                    dtype=np.uint32)


def windows_from_bits(block: np.ndarray, T: int, k: int, L: int) -> np.ndarray:
    """All T windows of one block, read from the unpacked bit array."""
    bits = block_bits(block, T, k)
    return np.array([_lib.oracle_window_from_bits(_p(bits, _u8p), T, k, L, t) for t in range(T)],
                    dtype=np.uint32)


def expand(codes: np.ndarray, scales: np.ndarray, lut: np.ndarray, axis: int, T: int, L: int,
           k: int, in_features: int, out_features: int, block_interleave: int = 0) -> np.ndarray:
    """Decoded bf16 weights (uint16 bits), shape [rows, cols]; `codes` in the
    layout `block_interleave` names (0 row-major, 2 block pairs)."""
    rows, cols = _dims(axis, in_features, out_features)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    lut = np.ascontiguousarray(lut, dtype=np.float32)
    assert codes.size == rows * cols * k // 32 and scales.size == rows and lut.size == 1 << L
    W = np.empty((rows, cols), dtype=np.uint16)
    ok = _lib.oracle_expand(_p(codes, _u32p), _p(scales, _f32p), _p(lut, _f32p), axis, T, L, k,
                            in_features, out_features, block_interleave, _p(W, _u16p))
    if not ok:
        raise ValueError("oracle_expand: unsupported geometry")
    return W


def matmul_f64(x: np.ndarray, W: np.ndarray, axis: int, in_features: int,
               out_features: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    M = x.shape[0]
    assert x.shape == (M, in_features)
    y = np.empty((M, out_features), dtype=np.float64)
    _lib.oracle_matmul_f64(_p(x, _u16p), M, _p(W, _u16p), axis, in_features, out_features,
                           _p(y, _f64p))
    return y


def fused_f64(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, lut: np.ndarray, axis: int,
              T: int, L: int, k: int, in_features: int, out_features: int,
              n_begin: int = 0, n_end: int | None = None, block_interleave: int = 0) -> np.ndarray:
    """y (float64, [M, out_features]); only output columns [n_begin, n_end) are
    computed, the others are left at zero. `codes` in the layout
    `block_interleave` names (0 row-major, 2 block pairs)."""
    if n_end is None:
        n_end = out_features
    x = np.ascontiguousarray(x, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    lut = np.ascontiguousarray(lut, dtype=np.float32)
    M = x.shape[0]
    y = np.zeros((M, out_features), dtype=np.float64)
    ok = _lib.oracle_fused_f64(_p(x, _u16p), M, _p(codes, _u32p), _p(scales, _f32p),
                               _p(lut, _f32p), axis, T, L, k, in_features, out_features,
                               block_interleave, n_begin, n_end, _p(y, _f64p))
    if not ok:
        raise ValueError("oracle_fused_f64: unsupported geometry")
    return y


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns exactly (a bit shift, no rounding)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def interleave_blocks(codes: np.ndarray, rows: int, nb: int, wpb: int) -> np.ndarray:
    """Row-major codes [rows][nb][wpb] rewritten in the block-interleave-2
    order: block pairs outermost, then rows, then the pair's two blocks
    ([P60] vector-expand.ts and [P59] scatter.ts address a block so when
    INTERLEAVE is set). A reshape and a transpose; nb must be even."""
    if nb % 2:
        raise ValueError("block interleave 2 needs an even number of blocks per row")
    a = np.asarray(codes, dtype=np.uint32).reshape(rows, nb // 2, 2, wpb)
    return np.ascontiguousarray(a.transpose(1, 0, 2, 3)).reshape(-1)


def deinterleave_blocks(codes: np.ndarray, rows: int, nb: int, wpb: int) -> np.ndarray:
    """Inverse of interleave_blocks."""
    if nb % 2:
        raise ValueError("block interleave 2 needs an even number of blocks per row")
    a = np.asarray(codes, dtype=np.uint32).reshape(nb // 2, rows, 2, wpb)
    return np.ascontiguousarray(a.transpose(1, 0, 2, 3)).reshape(-1)


def silu(v: float) -> float:
    """silu(v) = v / (1 + exp(-v)) in double."""
    return float(_lib.oracle_silu(v))


def swiglu_f64(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u elementwise in double (the SwiGLU of an MLP's gate and
    up projection outputs); g and u of the same shape."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    if g.shape != u.shape:
        raise ValueError("gate and up outputs differ in shape")
    h = np.empty_like(g)
    _lib.oracle_swiglu_f64(_p(g, _f64p), _p(u, _f64p), g.size, _p(h, _f64p))
    return h


def mlp_up_swiglu_f64(x: np.ndarray, gate, up, T: int, L: int, k: int, in_features: int,
                      out_features: int, n_begin: int = 0, n_end: int | None = None,
                      block_interleave: int = 0) -> np.ndarray:
    """h = silu(x Wg^T) * (x Wu^T) in double, [M, out_features]: gate and up
    are (codes, scales, lut) of two axis-1 projections of one geometry; only
    output columns [n_begin, n_end) are computed, the others are zero."""
    g = fused_f64(x, *gate, 1, T, L, k, in_features, out_features, n_begin, n_end,
                  block_interleave)
    u = fused_f64(x, *up, 1, T, L, k, in_features, out_features, n_begin, n_end,
                  block_interleave)
    return swiglu_f64(g, u)
