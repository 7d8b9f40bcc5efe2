"""Bit-field decoders of the two number formats of the FP4 KV cache (oracle).

Test infrastructure only (see the package docstring).

The pages name the formats without spelling them out: the main KV "quantises
to E2M1 with one E4M3 scale per 16 channels", following NVFP4 without its
global scale (ai-maestro.online, "FP4 KV, Bounded Replay, and other
extensions").  Their bit layouts are the public OCP 8-bit / MX definitions:

* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
  subnormal (value = m * 0.5).  No infinities or NaNs.  Magnitudes of codes
  0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 (OCP "E4M3FN", the NVFP4 scale type): 1 sign bit, 4 exponent bits
  (bias 7), 3 mantissa bits; exponent 0 is subnormal (value = m/8 * 2^-6);
  S.1111.111 is NaN; no infinities; largest finite value 448.
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    code &= 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                      # subnormal: m * 2^(1-bias) * 2^-1
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Value of an 8-bit OCP E4M3FN code (NaN for 0x7F / 0xFF)."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)   # subnormal
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite E4M3 codes 0x00..0x7E in ascending value order
# (zero plus 126 positive values: "127 positive finite scales" counting zero).
E4M3_FINITE_CODES = np.arange(0x7F, dtype=np.int64)
E4M3_GRID = E4M3[:0x7F].copy()
E4M3_MAX = 448.0
E2M1_GRID = E2M1[:8].copy()        # magnitudes of codes 0..7
E2M1_MAX = 6.0


def dequant_rows(codes: np.ndarray, scales: np.ndarray, dim: int) -> np.ndarray:
    """FP64 values of FP4 rows: value[c] = E2M1(nibble c) * E4M3(scale of c // 16).

    ``codes`` [n, dim/2] uint8 with the even channel in the low nibble,
    ``scales`` [n, dim/16] uint8.  Exact in FP64."""
    codes = np.asarray(codes, dtype=np.uint8)[:, : dim // 2]
    scales = np.asarray(scales, dtype=np.uint8)[:, : dim // 16]
    n = codes.shape[0]
    nib = np.empty((n, dim), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    vals = E2M1[nib]
    s = np.repeat(E4M3[scales], 16, axis=1)
    return vals * s
