"""8-bit sliding-window cache rows: E4M3 codes with one power-of-two scale per
row (oracle, FP64).

Test infrastructure only (see the package docstring).

Pages: the sliding-window cache keeps 8-bit precision while the main KV
moves to FP4 (kongchang.com, "Three Core Innovations"); the previous model's
cache was FP8 (ai-maestro.online, "FP4 KV, Bounded Replay, and other
extensions").  The pages do not give the 8-bit format.  Readings taken:

* R26 the codes are OCP E4M3FN, the 8-bit format the FP4 cache already uses
      for its scales;
* R27 one scale per row (one token's d-vector), a power of two 2^k with the
      smallest integer k such that max|x| <= 448 * 2^k (k = 0 for an
      all-zero row).  Dividing by a power of two is exact, so each code is
      a single rounding;
* R28 code = E4M3(|x| / 2^k) to nearest, ties to the even code (|x| / 2^k
      never exceeds 448, so nothing saturates), sign bit = sign bit of x;
* the value of a code is E4M3(code) * 2^k, exact in FP64.

The rounding is evaluated exactly: |x| / 2^k is an exact FP64 number and is
compared with the exact midpoints between neighbouring E4M3 values.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3, E4M3_GRID, E4M3_MAX
from .quant import _round_half_even_index

_E4M3_MID = 0.5 * (E4M3_GRID[:-1] + E4M3_GRID[1:])           # 126 exact midpoints


def row_exponents(x: np.ndarray) -> np.ndarray:
    """k per row: the smallest integer with max|x| <= 448 * 2^k (R27)."""
    amax = np.abs(np.asarray(x, dtype=np.float64)).max(axis=1)
    k = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # a first guess from log2, then exact corrections by comparison
    k[nz] = np.ceil(np.log2(amax[nz] / E4M3_MAX)).astype(np.int64)
    for _ in range(2):
        up = nz & (E4M3_MAX * np.ldexp(1.0, k) < amax)
        k[up] += 1
        down = nz & (E4M3_MAX * np.ldexp(1.0, k - 1) >= amax)
        k[down] -= 1
    return k


def quantize_swa_rows(x: np.ndarray):
    """Rows x [n, d] (float values, e.g. bf16 inputs) -> (codes [n, d] uint8,
    scales [n] float64 powers of two)."""
    x = np.asarray(x, dtype=np.float64)
    k = row_exponents(x)
    scale = np.ldexp(1.0, k)
    y = np.abs(x) / scale[:, None]                               # exact
    mag = _round_half_even_index(y, _E4M3_MID)                   # 0 .. 126
    sign = np.signbit(x).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8), scale


def swa_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP64 values of 8-bit window rows: E4M3(code) * scale of the row."""
    return E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[..., None]
