"""Seeded synthetic inputs for the trellis dequantize-and-multiply workloads.

This module only draws random numbers. It holds none of the method's
arithmetic (no window extraction, no codebook lookup, no scaling, no
contraction), so that the HIP path and the CPU oracle can both be fed from it
without sharing any decoding code.

Recipe (one numpy PCG64 stream per tensor, seeded with
``[config_id, k, M, projection, tensor_id]``):

* codes   (tensor 0): uniform random u32 words, ``rows x (cols*k/32)``;
* LUT     (tensor 1): 4096 float32 draws from N(0, 1);
* scales  (tensor 2): ``rows`` float32 draws from U[0.5, 1.5);
* x       (tensor 3): ``M x in_features`` N(0, 1) draws, float32, then
  rounded to bfloat16 (round-to-nearest-even, by torch's CPU cast) and kept
  as raw uint16 bit patterns.

Shapes follow the storage convention of the method: the stored matrix is
``[rows, cols]``; on axis 1 ``rows = out_features`` and ``cols =
in_features``; on axis 0 ``rows = in_features`` and ``cols = out_features``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

LUT_ENTRIES = 4096

# Workload identifiers used as the first seed word.
CONFIG_IDS = {
    "tiny_gemv": 0,          # axis 1, in 512 -> out 256, M 1
    "qwen_up_gemv": 1,       # axis 1, in 5120 -> out 17408, M 1
    "qwen_down_scatter": 2,  # axis 0, in 17408 -> out 5120, M 1
    "qwen_up_prefill": 3,    # axis 1, in 5120 -> out 17408, M 5..32
    "qwen_mlp": 4,           # gate/up axis 1 + down axis 0, k 4
    "test": 99,              # small ad-hoc test problems
}


@dataclass(frozen=True)
class Shape:
    """Storage shape of one trellis-coded projection."""

    axis: int
    T: int
    L: int
    k: int
    in_features: int
    out_features: int
    block_interleave: int = 0  # code layout: 0 row-major, 2 block pairs

    @property
    def rows(self) -> int:
        return self.out_features if self.axis == 1 else self.in_features

    @property
    def cols(self) -> int:
        return self.in_features if self.axis == 1 else self.out_features

    @property
    def words_per_row(self) -> int:
        return self.cols * self.k // 32


def _rng(cfg: int, k: int, M: int, proj: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([cfg, k, M, proj, tensor])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) using torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def codes(shape: Shape, cfg: int, M: int = 1, proj: int = 0) -> np.ndarray:
    g = _rng(cfg, shape.k, M, proj, 0)
    return g.integers(0, 2**32, size=(shape.rows, shape.words_per_row), dtype=np.uint32)


def lut(shape: Shape, cfg: int, M: int = 1, proj: int = 0) -> np.ndarray:
    g = _rng(cfg, shape.k, M, proj, 1)
    return g.standard_normal(1 << shape.L).astype(np.float32)


def scales(shape: Shape, cfg: int, M: int = 1, proj: int = 0) -> np.ndarray:
    g = _rng(cfg, shape.k, M, proj, 2)
    return g.uniform(0.5, 1.5, shape.rows).astype(np.float32)


def activations(shape: Shape, cfg: int, M: int = 1, proj: int = 0) -> np.ndarray:
    g = _rng(cfg, shape.k, M, proj, 3)
    return to_bf16_bits(g.standard_normal((M, shape.in_features)).astype(np.float32))


@dataclass
class Problem:
    shape: Shape
    M: int
    codes: np.ndarray    # uint32 [rows, cols*k/32]
    lut: np.ndarray      # float32 [4096]
    scales: np.ndarray   # float32 [rows]
    x: np.ndarray        # uint16 (bf16 bits) [M, in_features]


def make_problem(shape: Shape, M: int, cfg: int, proj: int = 0) -> Problem:
    return Problem(shape, M, codes(shape, cfg, M, proj), lut(shape, cfg, M, proj),
                   scales(shape, cfg, M, proj), activations(shape, cfg, M, proj))


def integer_lut(L: int = 12) -> np.ndarray:
    """Codebook of small integers, (i mod 15) - 7: every product with a
    scale in {0.5, 1, 2} and a small-integer activation is exact in float32."""
    return ((np.arange(1 << L) % 15) - 7).astype(np.float32)


def one_hot_x(M: int, n: int, cols: list[int]) -> np.ndarray:
    """bf16 bit patterns of M one-hot activation rows (row m is e_{cols[m]})."""
    x = np.zeros((M, n), dtype=np.float32)
    for m, c in enumerate(cols):
        x[m, c] = 1.0
    return to_bf16_bits(x)
