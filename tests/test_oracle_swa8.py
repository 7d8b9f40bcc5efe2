"""Pins of the oracle's 8-bit sliding-window rows (oracle/swa8.py): the E4M3
rounding against torch's float8_e4m3fn cast (a library routine: round to
nearest even), the per-row power-of-two scale rule, exact round trips, and
signed zeros."""
import numpy as np
import pytest
import torch

from oracle import swa8
from oracle.formats import E4M3, E4M3_GRID


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_values() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v) & (np.abs(v) <= 448.0)]


def test_codes_match_torch_cast_for_every_bf16_value():
    v = _bf16_values()
    rows = np.stack([np.full(v.shape, 448.0, dtype=np.float32), v], axis=1)   # amax 448 -> scale 1
    codes, scales = swa8.quantize_swa_rows(rows)
    assert (scales == 1.0).all()
    np.testing.assert_array_equal(codes[:, 1], _torch_e4m3(v))


def test_codes_at_and_around_every_midpoint():
    mids = 0.5 * (E4M3_GRID[:-1] + E4M3_GRID[1:])
    m32 = mids.astype(np.float32)
    assert (m32.astype(np.float64) == mids).all()                   # midpoints are exact in fp32
    vals = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1000))])
    vals = np.concatenate([vals, -vals])
    rows = np.stack([np.full(vals.shape, 448.0, dtype=np.float32), vals], axis=1)
    codes, _ = swa8.quantize_swa_rows(rows)
    np.testing.assert_array_equal(codes[:, 1], _torch_e4m3(vals))


def test_row_scale_is_the_smallest_power_of_two_covering_the_row():
    rng = np.random.default_rng(3)
    amax = np.concatenate([
        448.0 * np.ldexp(1.0, np.arange(-20, 10)),                      # exact boundaries
        np.nextafter(448.0 * np.ldexp(1.0, np.arange(-20, 10)), np.inf),
        np.nextafter(448.0 * np.ldexp(1.0, np.arange(-20, 10)), 0.0),
        np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-6, 6, 200),
    ])
    rows = np.stack([amax * np.where(np.arange(len(amax)) % 2 == 0, 1, -1), amax * 0.25], axis=1)
    k = swa8.row_exponents(rows)
    assert (amax <= 448.0 * np.ldexp(1.0, k)).all()
    assert (amax > 448.0 * np.ldexp(1.0, k - 1)).all()
    assert swa8.row_exponents(np.zeros((1, 4)))[0] == 0


@pytest.mark.parametrize("k", [-12, -7, 0, 5])
def test_exact_values_round_trip(k):
    rng = np.random.default_rng(100 + k)
    c = rng.integers(0, 127, size=(64, 32))
    sign = rng.integers(0, 2, size=(64, 32))
    x = np.where(sign == 1, -1.0, 1.0) * E4M3_GRID[c] * np.ldexp(1.0, k)
    x[:, 0] = 448.0 * np.ldexp(1.0, k)                             # fixes the row scale at 2^k
    codes, scales = swa8.quantize_swa_rows(x)
    assert (scales == np.ldexp(1.0, k)).all()
    np.testing.assert_array_equal(swa8.swa_values(codes, scales), x)
    want = (np.where(sign == 1, 0x80, 0) | c).astype(np.uint8)
    want[:, 0] = 0x7E
    np.testing.assert_array_equal(codes[:, 1:][c[:, 1:] > 0], want[:, 1:][c[:, 1:] > 0])


def test_signed_zeros_and_values_below_half_the_smallest_step():
    x = np.array([[448.0, -0.0, 0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.5, -(2.0 ** -11)]])
    codes, scales = swa8.quantize_swa_rows(x)
    assert scales[0] == 1.0
    # 2^-10 is half-way between 0 and 2^-9: ties go to the even code 0
    np.testing.assert_array_equal(codes[0], [0x7E, 0x80, 0x00, 0x00, 0x80, 0x01, 0x80])
    assert E4M3[0x80] == 0.0
