"""Pins of the oracle's FP4 quantiser (CPU only).

The oracle decides roundings by exact threshold comparisons.  These tests pin
it to an independent brute force (nearest grid value by exact rational
distance, ties to the even code), to exhaustive round trips over every scale
and every code, to every scale midpoint and its fp32 neighbours, and to
torch's float32 -> float8_e4m3fn cast away from midpoints."""
import itertools
from fractions import Fraction

import numpy as np
import torch

from oracle import formats, quant

E4M3_FR = [Fraction(formats.e4m3_value(c)) for c in range(0x7F)]
E2M1_FR = [Fraction(formats.e2m1_value(c)) for c in range(8)]


def nearest_even(y: Fraction, grid):
    """Brute force: index of the grid value nearest to y; ties -> even index."""
    best = None
    for i, v in enumerate(grid):
        d = abs(y - v)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0 and best[1] % 2 == 1):
            best = (d, i)
    return best[1]


def brute_quantize_group(xs):
    amax = max(abs(Fraction(float(x))) for x in xs)
    sc = nearest_even(amax / 6, E4M3_FR)
    s = E4M3_FR[sc]
    codes = []
    for x in xs:
        sign = 8 if np.signbit(x) else 0
        if s == 0:
            codes.append(sign)
        else:
            codes.append(sign | nearest_even(abs(Fraction(float(x))) / s, E2M1_FR))
    return sc, codes


def oracle_group(xs):
    codes, sc = quant.quantize_rows(np.asarray(xs, dtype=np.float32)[None, :])
    nib = np.empty(16, dtype=np.int64)
    nib[0::2] = codes[0] & 0xF
    nib[1::2] = codes[0] >> 4
    return int(sc[0, 0]), [int(v) for v in nib]


def test_brute_force_random_groups():
    rng = np.random.default_rng(7)
    for t in range(300):
        scale = 10.0 ** rng.uniform(-4, 3.5)
        xs = (rng.standard_normal(16) * scale).astype(np.float32)
        if t % 5 == 0:   # put elements exactly on E2M1 midpoints of the group's scale
            sc, _ = brute_quantize_group(xs)
            s = float(E4M3_FR[sc])
            mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
            for k in range(1, 8):
                xs[k] = np.float32(mids[k - 1] * s * (1 if k % 2 else -1))
        assert oracle_group(xs) == brute_quantize_group(xs), xs


def test_exhaustive_round_trip_every_scale_and_code():
    # amax = 6 s makes the scale exactly s; every element E2M1(c) * s must map back to c
    for sc in range(1, 0x7F):
        s = formats.e4m3_value(sc)
        for c in range(16):
            xs = np.zeros(16, dtype=np.float32)
            xs[0] = np.float32(6.0 * s)
            xs[1] = np.float32(formats.e2m1_value(c) * s)
            if c == 8:
                xs[1] = np.float32(-0.0)
            got_sc, got = oracle_group(xs)
            assert got_sc == sc, (sc, c)
            assert got[0] == 7 and got[1] == c, (sc, c, got[:2])


def test_scale_midpoints_and_neighbours():
    n_cases = 0
    for c in range(0x7E):
        mid6 = 3.0 * (formats.e4m3_value(c) + formats.e4m3_value(c + 1))   # exact in fp32
        for amax in (np.nextafter(np.float32(mid6), np.float32(0)), np.float32(mid6),
                     np.nextafter(np.float32(mid6), np.float32(np.inf))):
            xs = np.zeros(16, dtype=np.float32)
            xs[3] = amax
            got_sc, _ = oracle_group(xs)
            want_sc, _ = brute_quantize_group(xs)
            assert got_sc == want_sc, (c, float(amax))
            n_cases += 1
    assert n_cases == 126 * 3


def test_element_midpoints_every_scale():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sc in range(1, 0x7F):
        s = formats.e4m3_value(sc)
        for m in mids:
            t = np.float32(m * s)
            xs = np.zeros(16, dtype=np.float32)
            xs[0] = np.float32(6.0 * s)
            xs[1:4] = [np.nextafter(t, np.float32(0)), t, np.nextafter(t, np.float32(np.inf))]
            xs[4:7] = -xs[1:4]
            assert oracle_group(xs) == brute_quantize_group(xs), (sc, m)


def test_saturation_zero_and_signs():
    xs = np.zeros(16, dtype=np.float32)
    xs[0] = 1e6                          # amax/6 >> 448 -> scale 448 (0x7E)
    xs[1] = -7.0 * 448
    sc, c = oracle_group(xs)
    assert sc == 0x7E and c[0] == 7 and c[1] == 15
    # all-zero group: scale 0, codes keep the sign of zero
    xs = np.array([0.0, -0.0] * 8, dtype=np.float32)
    sc, c = oracle_group(xs)
    assert sc == 0 and c == [0, 8] * 8
    # amax/6 exactly 2^-10 is a tie between 0 and 2^-9 -> even code 0 -> zero group
    xs = np.zeros(16, dtype=np.float32)
    xs[0] = np.float32(6 * 2.0 ** -10)
    xs[1] = -np.float32(1e-5)
    sc, c = oracle_group(xs)
    assert sc == 0 and c[0] == 0 and c[1] == 8
    # just above the tie -> smallest subnormal scale 2^-9
    xs[0] = np.nextafter(np.float32(6 * 2.0 ** -10), np.float32(1))
    assert oracle_group(xs)[0] == 1
    # scale rounded below amax/6 -> largest element saturates at 6.0 (code 7)
    s = formats.e4m3_value(0x38)            # 1.0; next value is 1.125
    xs = np.zeros(16, dtype=np.float32)
    xs[0] = np.float32(6.0 * 1.06)          # amax/6 = 1.06 rounds to 1.0
    sc, c = oracle_group(xs)
    assert sc == 0x38 and c[0] == 7 and s == 1.0


def test_scale_matches_torch_cast_off_midpoints():
    rng = np.random.default_rng(3)
    amax = (10.0 ** rng.uniform(-3, 3.4, size=5000)).astype(np.float32)
    y32 = (amax.astype(np.float64) / 6.0).astype(np.float32)
    mids = 0.5 * (formats.E4M3_GRID[:-1] + formats.E4M3_GRID[1:])
    # skip inputs whose rounded quotient sits within 2 ulp of a midpoint
    near = np.min(np.abs(y32.astype(np.float64)[:, None] - mids[None, :]), axis=1) <= \
        2 * np.spacing(y32).astype(np.float64)
    keep = ~near & (y32 <= 448.0)
    torch_codes = torch.from_numpy(y32[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = quant.scale_codes(amax[keep])
    np.testing.assert_array_equal(ours, torch_codes)
    assert keep.sum() > 4000


def test_rows_pack_even_channel_low_nibble():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 6.0      # group 0 scale -> 1.0, channel 0 -> code 7
    x[0, 1] = -1.0     # channel 1 -> code 0xA
    codes, sc = quant.quantize_rows(x)
    assert codes[0, 0] == 0x7 | (0xA << 4)
    assert sc[0, 0] == 0x38 and sc[0, 1] == 0x00


def test_dequantised_error_bound():
    # |x - deq(x)| <= half an E2M1 step at the group's scale, except saturation
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    codes, sc = quant.quantize_rows(x)
    deq = formats.dequant_rows(codes, sc, 512)
    s = np.repeat(formats.E4M3[sc], 16, axis=1)
    err = np.abs(deq - x)
    assert np.all(err <= 1.0 * s + 1e-30)         # largest E2M1 gap is 2 (4 -> 6), half = 1
    # scales track amax/6 within E4M3 relative precision
    amax = np.abs(x.reshape(64, 32, 16)).max(axis=2)
    assert np.all(np.abs(formats.E4M3[sc] - amax / 6) <= amax / 6 * 2.0 ** -4 + 2.0 ** -10)


def test_itertools_small_grid_exhaustive():
    # every combination of a few tricky magnitudes in a 2-element pattern
    vals = [0.0, -0.0, 2.0 ** -12, 0.1, 0.25, 1.0, 2.9999, 3.0, 5.0, 6.0, 449.0 * 6, 1e9]
    for a, b in itertools.product(vals, repeat=2):
        xs = np.zeros(16, dtype=np.float32)
        xs[0], xs[9] = a, -b if b else b
        assert oracle_group(xs) == brute_quantize_group(xs), (a, b)
