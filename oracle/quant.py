"""FP4 quantiser of the main KV cache (oracle, FP64).

Test infrastructure only (see the package docstring).

What the pages fix: each main-cache entry is stored as 4-bit E2M1 values,
every run of 16 channels sharing one 8-bit E4M3 multiplier -- the NVFP4
layout without its tensor-wide factor (ai-maestro.online, "FP4 KV, Bounded
Replay, and other extensions"; wpnews.pro, "What is Compressed Sparse
Attention 2 CSA2?"; cutthecrap, "Architectural Breakthroughs").

The pages give no formula; the readings taken for what they leave open:

* R2  a scale group is 16 consecutive channels of one entry;
* R3  scale = E4M3(amax / 6) rounded to nearest, ties to the even code
      (the NVFP4 block rule with the global factor fixed at 1);
* R4  amax / 6 above 448 saturates to 448 (code 0x7E); never NaN;
* R5  a zero scale (amax/6 <= 2^-10, the half-way point to the smallest
      subnormal) makes every code of the group a signed zero;
* R6  element code = E2M1(|x| / scale) rounded to nearest, ties to the even
      code, saturating at 6;
* R7  the sign bit is the sign bit of x (also for -0.0 and negative values
      that round to zero);
* R8  two codes per byte, the even channel in the low nibble.

"Round to nearest, ties to even" is evaluated exactly: y = amax/6 is
compared with the midpoints mu between neighbouring E4M3 values through
amax <-> 6*mu, and r = |x|/s with the E2M1 midpoints m through |x| <-> m*s.
All of 6*mu, m*s, amax and |x| are exact FP64 numbers, so no quotient is
ever rounded and no tie is invented or lost.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_GRID, E4M3_GRID

GROUP = 16
# midpoints between neighbouring non-negative finite E4M3 values, times 6
_E4M3_MID6 = 3.0 * (E4M3_GRID[:-1] + E4M3_GRID[1:])          # 126 values, exact
# midpoints between neighbouring E2M1 magnitudes: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
_E2M1_MID = 0.5 * (E2M1_GRID[:-1] + E2M1_GRID[1:])


def _round_half_even_index(value: np.ndarray, scaled_mids: np.ndarray) -> np.ndarray:
    """Index of the nearest grid point to ``value`` given the sorted midpoints
    between neighbouring grid points; an exact tie picks the even index.
    Values above the last midpoint map to the last grid point (saturation)."""
    n = scaled_mids.shape[0]
    below = np.searchsorted(scaled_mids, value, side="left")      # #mids strictly below
    tie = (below < n) & (scaled_mids[np.minimum(below, n - 1)] == value)
    return below + (tie & (below % 2 == 1))


def scale_codes(amax: np.ndarray) -> np.ndarray:
    """E4M3 code (0x00..0x7E) of amax/6, nearest-even, saturating (R3, R4, R5)."""
    return _round_half_even_index(np.asarray(amax, dtype=np.float64), _E4M3_MID6).astype(np.uint8)


def element_codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes of x / s per element (R6, R7); s broadcasts over x."""
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    a = np.abs(x)
    mids = _E2M1_MID[None, :] * s.reshape(-1, 1)                  # exact products
    mag = np.empty(a.size, dtype=np.int64)
    af = a.reshape(-1)
    below = (mids < af[:, None]).sum(axis=1)
    at = np.minimum(below, len(_E2M1_MID) - 1)
    tie = (below < len(_E2M1_MID)) & (mids[np.arange(af.size), at] == af)
    mag[:] = below + (tie & (below % 2 == 1))
    mag = mag.reshape(a.shape)
    mag = np.where(s == 0.0, 0, mag)                              # R5
    sign = np.signbit(x).astype(np.int64) << 3                    # R7
    return (mag | sign).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """Quantise fp32 rows [n, d] (d % 16 == 0) to (codes [n, d/2], scales [n, d/16]).

    Per row and per 16-channel group: amax -> E4M3 scale of amax/6 -> E2M1 code
    of each x/scale -> pack two codes per byte, even channel low (R8)."""
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape
    assert d % GROUP == 0
    g = x.astype(np.float64).reshape(n, d // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    sc = scale_codes(amax)                                        # [n, d/16]
    s = E4M3_GRID[sc.astype(np.int64)]
    nib = element_codes(g, s[:, :, None]).reshape(n, d)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, sc
