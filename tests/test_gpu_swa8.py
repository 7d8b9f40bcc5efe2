"""8-bit sliding-window rows on the GPU: csa2_quantize_swa_fp8 bit-exact
against the oracle (oracle/swa8.py), and csa2_sparse_attn reading such a
window (swa_fp8) against the FP64 oracle on the dequantised values."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from oracle import attention as oattn
from oracle import swa8
from tests.parity import ATTN_TOL, bf16_values, dev, host, rownorm_err
from fp4_kv_cache_e4m3_amd import synth
from tests.test_gpu_attn import CASES, make_case

pytestmark = pytest.mark.gpu


def gpu_quantize_swa(bits: np.ndarray):
    rows, d = bits.shape
    out = torch.full((rows, d), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    csa2.quantize_swa_fp8(dev(np.ascontiguousarray(bits).view(np.int16)), out, sc)
    return host(out), host(sc)


def check_rows(bits: np.ndarray):
    codes, sc = gpu_quantize_swa(bits)
    rc, rs = swa8.quantize_swa_rows(bf16_values(bits))
    np.testing.assert_array_equal(codes, rc)
    np.testing.assert_array_equal(sc, rs.astype(np.float32))


@pytest.mark.parametrize("dim", [512, 128])
def test_quantize_every_bf16_value(dim):
    """Every bf16 value with magnitude in [2^-100, 2^100] (and both zeros),
    shuffled into rows, so each row gets its own scale."""
    b = np.arange(1 << 16, dtype=np.uint16)
    e = (b >> 7) & 0xFF
    keep = ((e >= 127 - 100) & (e <= 127 + 99)) | ((b & 0x7FFF) == 0)
    vals = np.random.default_rng(dim).permutation(b[keep])
    n = len(vals) // dim * dim
    check_rows(vals[:n].reshape(-1, dim))


def test_quantize_edge_rows():
    """Zero and negative-zero rows; rows whose maximum is exactly 448 * 2^k
    and the next bf16 value above it (the scale moves to 2^(k+1))."""
    from fp4_kv_cache_e4m3_amd import synth
    d = 512
    rng = np.random.default_rng(1)
    rows = [np.zeros(d, np.uint16), np.full(d, 0x8000, np.uint16)]
    for k in (-20, -7, 0, 7, 30):
        r = synth.f32_to_bf16_bits(rng.standard_normal(d).astype(np.float32) * np.float32(2.0 ** k))
        r[3] = synth.f32_to_bf16_bits(np.array([448.0 * 2.0 ** k], np.float32))[0]
        rows.append(r)
        r2 = r.copy()
        r2[3] += 1                                          # the next bf16 value above
        rows.append(r2)
    check_rows(np.stack(rows))


SWA8_CASES = [CASES[i] for i in (0, 1, 2, 3, 4, 5, 6, 9, 10)]


def run_case(case, swa_len=None, kill=None):
    B, Qn, T, d, H, W, k = case
    codes, scales, q, swa, topk = make_case(sum(case) + 1, B, Qn, T, d, H, W, k, fill=None)
    if kill is not None:
        topk[kill] = -1
    rows = swa.reshape(-1, d)
    c8, s8 = gpu_quantize_swa(rows)
    rc, rs = swa8.quantize_swa_rows(bf16_values(rows))
    np.testing.assert_array_equal(c8, rc)
    np.testing.assert_array_equal(s8, rs.astype(np.float32))
    nq = B * Qn
    q_d = dev(q.view(np.int16))
    t_d = dev(topk.astype(np.int32)) if topk.shape[1] > 0 else None
    sw_d = dev(c8.reshape(swa.shape)) if W > 0 else None
    sc_d = dev(s8.reshape(swa.shape[:2]).astype(np.float32)) if W > 0 else None
    sl_d = dev(np.asarray(swa_len, np.int32)) if swa_len is not None else None
    out = torch.full((nq, H, d), float("nan"), dtype=torch.float32, device="cuda")
    # the argument struct holds raw pointers: keep every device buffer alive
    # until the call (a temporary's block could be handed to the workspace)
    c_d, s_d = dev(codes), dev(scales)
    args = csa2.attn_args(q_d, c_d, s_d, t_d, sw_d, out, Qn, T, W, sl_d,
                          swa_scale=sc_d if W > 0 else None)
    n = csa2.attn_workspace_size(args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None
    csa2.sparse_attn(args, ws)
    got = host(out)
    swa_vals = swa8.swa_values(rc, rs).reshape(swa.shape)
    ref = oattn.sparse_attn(bf16_values(q), codes, scales, topk, swa_vals, Qn, T, window=W, swa_len=swa_len)
    return got, ref


@pytest.mark.parametrize("case", SWA8_CASES, ids=lambda c: "B{}Q{}T{}d{}H{}W{}k{}".format(*c))
def test_attn_with_8bit_window_matches_oracle(case):
    got, ref = run_case(case)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_with_8bit_partial_window():
    case = (3, 2, 400, 512, 16, 128, 512)
    got, ref = run_case(case, swa_len=[129, 5, 0], kill=[1, 4, 5])
    assert np.all(got[4:6] == 0.0)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_quantize_into_newest_window_slots():
    """A decode step's new rows go straight into slot R-1 of every sequence's
    window (rows strided by R * d bytes, scales by R): bit-exact against the
    oracle, every other slot untouched."""
    B, R, d = 5, 128, 512
    rng = np.random.default_rng(77)
    bits = synth.f32_to_bf16_bits((rng.standard_normal((B, d)) * 3).astype(np.float32))
    codes = torch.full((B, R, d), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((B, R), float("nan"), dtype=torch.float32, device="cuda")
    csa2.quantize_swa_fp8(dev(bits.view(np.int16)), codes[:, R - 1, :], sc[:, R - 1])
    got_c, got_s = host(codes), host(sc)
    rc, rs = swa8.quantize_swa_rows(bf16_values(bits))
    np.testing.assert_array_equal(got_c[:, R - 1], rc)
    np.testing.assert_array_equal(got_s[:, R - 1], rs.astype(np.float32))
    assert np.all(got_c[:, :R - 1] == 0xA5) and np.all(np.isnan(got_s[:, :R - 1]))
