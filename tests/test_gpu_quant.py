"""GPU parity of csa2_quantize_kv / csa2_dequantize_kv against the oracle:
bit-exact codes and scales, exact dequantised values."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_e4m3_amd import synth
import fp4_kv_cache_e4m3_amd as csa2
from oracle import formats, quant
from tests.parity import dev, host

pytestmark = pytest.mark.gpu


def gpu_quantize(x: np.ndarray):
    n, d = x.shape
    codes = torch.empty((n, d // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, d // 16), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(dev(x), codes, scales)
    return host(codes), host(scales)


def exhaustive_groups() -> np.ndarray:
    """Every scale x every code, every scale midpoint and its fp32 neighbours,
    every element midpoint at every scale, saturation, zeros and signed zeros."""
    groups = []
    for sc in range(1, 0x7F):
        s = formats.e4m3_value(sc)
        for c in range(16):
            g = np.zeros(16, np.float32)
            g[0] = 6.0 * s
            g[1 + (c % 15)] = formats.e2m1_value(c) * s if c != 8 else -0.0
            groups.append(g)
        for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            t = np.float32(m * s)
            g = np.zeros(16, np.float32)
            g[0] = 6.0 * s
            g[1:4] = [np.nextafter(t, np.float32(0)), t, np.nextafter(t, np.float32(np.inf))]
            g[4:7] = -g[1:4]
            groups.append(g)
    for c in range(0x7E):
        mid6 = 3.0 * (formats.e4m3_value(c) + formats.e4m3_value(c + 1))
        for a in (np.nextafter(np.float32(mid6), np.float32(0)), np.float32(mid6),
                  np.nextafter(np.float32(mid6), np.float32(np.inf))):
            g = np.zeros(16, np.float32)
            g[5] = -a
            g[6] = a / 3
            groups.append(g)
    for special in ([1e6, -7 * 448.0], [0.0, -0.0], [6 * 2.0 ** -10, -1e-5], [6.0 * 1.06, 1.0]):
        g = np.zeros(16, np.float32)
        g[:2] = special
        groups.append(g)
    x = np.stack(groups)
    pad = (-len(x)) % 32
    x = np.concatenate([x, np.zeros((pad, 16), np.float32)])
    return x.reshape(-1, 512)


@pytest.mark.parametrize("copies", [1, 8])
def test_quantize_exhaustive_bit_exact(copies):
    """The exhaustive groups once (a small launch: four lanes per group) and
    tiled 8 times (past 8,192 groups: the one-thread-per-group kernel)."""
    x = np.concatenate([exhaustive_groups()] * copies)
    c, s = gpu_quantize(x)
    rc, rs = quant.quantize_rows(x)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("dim", [32, 128, 512])
def test_quantize_random_scales(dim):
    rng = np.random.default_rng(dim)
    x = (rng.standard_normal((3001, dim)) * 10.0 ** rng.uniform(-5, 4, size=(3001, 1))).astype(np.float32)
    c, s = gpu_quantize(x)
    rc, rs = quant.quantize_rows(x)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_quantize_c1_rows():
    w = synth.C1
    x = synth.kv_source(w, 0)
    c, s = gpu_quantize(x)
    rc, rs = quant.quantize_rows(x)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(s, rs)


def test_quantize_c2_sampled_rows():
    w = synth.C2
    for b, r0 in ((0, 0), (17, 30000), (31, w.kv_len - 4096)):
        x = synth.kv_source_rows(w, b, r0, 4096)
        c, s = gpu_quantize(x)
        rc, rs = quant.quantize_rows(x)
        np.testing.assert_array_equal(c, rc)
        np.testing.assert_array_equal(s, rs)


def test_quantize_strided_rows_into_cache():
    B, T, d = 5, 37, 512
    codes = torch.full((B * T, d // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((B * T, d // 16), 0xCD, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(2)
    x = rng.standard_normal((B, d)).astype(np.float32)
    csa2.quantize_kv(dev(x), codes[T - 1::T], scales[T - 1::T])
    hc, hs = host(codes), host(scales)
    rc, rs = quant.quantize_rows(x)
    np.testing.assert_array_equal(hc[T - 1::T], rc)
    np.testing.assert_array_equal(hs[T - 1::T], rs)
    mask = np.ones(B * T, bool)
    mask[T - 1::T] = False
    assert np.all(hc[mask] == 0xAB) and np.all(hs[mask] == 0xCD)


def test_dequantize_every_code_and_scale():
    # all 256 code bytes under every finite scale byte (both signs)
    scale_bytes = [b for b in range(256) if (b & 0x7F) != 0x7F]
    d = 512
    rows = []
    for sb in scale_bytes:
        codes = np.tile(np.arange(256, dtype=np.uint8), 1)          # 256 bytes = 512 channels
        rows.append((codes, np.full(32, sb, np.uint8)))
    c = np.stack([r[0] for r in rows])
    s = np.stack([r[1] for r in rows])
    out = torch.empty((len(rows), d), dtype=torch.float32, device="cuda")
    csa2.dequantize_kv(dev(c), dev(s), out)
    got = host(out)
    ref = formats.dequant_rows(c, s, d)
    np.testing.assert_array_equal(got, ref.astype(np.float32))
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def bf16_rows_every_finite_value() -> np.ndarray:
    """Every finite bf16 bit pattern (both signs, subnormals, zeros) once, in
    rows of 512: consecutive patterns share a group, so each value is coded
    against the scale its neighbours set; plus the exhaustive fp32 groups
    above, rounded to bf16 (scale midpoints and element midpoints at every
    scale)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = (bits & 0x7F80) != 0x7F80
    vals = (bits[finite] << 16).view(np.float32)
    pad = (-len(vals)) % 512
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 512)
    ex = exhaustive_groups()
    ex16 = ((ex.view(np.uint32) + 0x7FFF + ((ex.view(np.uint32) >> 16) & 1)) & 0xFFFF0000).view(np.float32)
    ex16 = np.where(np.isfinite(ex16), ex16, np.float32(0))
    return np.concatenate([vals, ex16])


@pytest.mark.parametrize("copies", [1, 8])
def test_quantize_bf16_every_value_bit_exact(copies):
    """csa2_quantize_kv_bf16: bit-exact against the oracle on the widened
    values, through both kernels (small launch and the bulk kernel past 8,192
    groups)."""
    x = np.concatenate([bf16_rows_every_finite_value()] * copies)
    xb = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    assert torch.equal(xb.float().cpu(), torch.from_numpy(x))       # the rows are bf16 values
    n, d = x.shape
    codes = torch.empty((n, d // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, d // 16), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(xb, codes, scales)
    rc, rs = quant.quantize_rows(x)
    np.testing.assert_array_equal(host(scales), rs)
    np.testing.assert_array_equal(host(codes), rc)


@pytest.mark.parametrize("dim", [32, 512])
def test_quantize_bf16_strided_rows_into_cache(dim):
    """Strided bf16 source rows (a view) into strided cache rows, against the
    oracle; the cache rows in between stay untouched."""
    B, T = 7, 23
    rng = np.random.default_rng(dim + 1)
    src = torch.from_numpy((rng.standard_normal((B, dim + 64)) * 10.0 ** rng.uniform(-6, 5, (B, 1)))
                           .astype(np.float32)).to("cuda").to(torch.bfloat16)
    x = src[:, 8:8 + dim]                                             # row stride dim + 64, offset 16 bytes
    codes = torch.full((B * T, dim // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((B * T, dim // 16), 0xCD, dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(x, codes[T - 1::T], scales[T - 1::T])
    hc, hs = host(codes), host(scales)
    rc, rs = quant.quantize_rows(x.float().cpu().numpy())
    np.testing.assert_array_equal(hc[T - 1::T], rc)
    np.testing.assert_array_equal(hs[T - 1::T], rs)
    mask = np.ones(B * T, bool)
    mask[T - 1::T] = False
    assert np.all(hc[mask] == 0xAB) and np.all(hs[mask] == 0xCD)
