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


@pytest.mark.parametrize("case", [
    (3, 1, 1000, 512, 64, 128, 512, None),       # decode: one new row per sequence
    (2, 6, 900, 512, 16, 128, 300, None),        # 1 + 5 draft queries: six new rows
    (2, 3, 500, 128, 8, 64, 100, (2, 1)),        # d = 128, ring windows
    (1, 16, 700, 512, 16, 32, 64, (5,)),         # the most new rows the call takes, ring
], ids=lambda c: "B{}Q{}T{}d{}H{}W{}k{}ring{}".format(*c[:7], c[7] is not None))
@pytest.mark.parametrize("split", [(0, 0), (4, 1), (8, 3)], ids=["auto", "w4s1", "w8s3"])
def test_attn_encodes_new_window_rows(case, split):
    """swa_new: the attention call encodes the step's new window rows itself.
    Its output is bit-identical to the same call over a window whose newest
    rows already hold their 8-bit codes; afterwards the new rows' slots hold
    the oracle's codes and scales and every other slot is unchanged.  Work
    splits: the library's choice, 4-wave workgroups (four new rows per wave
    to encode), and three tile-list splits (only the first stores)."""
    B, Qn, T, d, H, W, k, ring = case
    waves, splits = split
    codes, scales, q, swa, topk = make_case(sum(case[:7]) + 3, B, Qn, T, d, H, W, k)
    R = swa.shape[1]                                    # W - 1 + Qn window rows
    rc, rs = swa8.quantize_swa_rows(bf16_values(swa.reshape(-1, d)))
    rc, rs = rc.reshape(B, R, d), rs.reshape(B, R).astype(np.float32)
    start = np.zeros(B, np.int32) if ring is None else np.asarray(ring, np.int32)
    full_c = np.stack([np.roll(rc[b], start[b], axis=0) for b in range(B)])     # row r in slot (r + start) % R
    full_s = np.stack([np.roll(rs[b], start[b]) for b in range(B)])
    new_slots = [(np.arange(R - Qn, R) + start[b]) % R for b in range(B)]
    stale_c, stale_s = full_c.copy(), full_s.copy()
    for b in range(B):
        stale_c[b, new_slots[b]] = 0xA5                 # the new rows' slots before the call
        stale_s[b, new_slots[b]] = np.nan
    new_bits = np.ascontiguousarray(swa[:, R - Qn:].reshape(B * Qn, d))

    def run(c8, s8, swa_new):
        out = torch.full((B * Qn, H, d), float("nan"), dtype=torch.float32, device="cuda")
        c_d, s_d = dev(c8), dev(s8)
        args = csa2.attn_args(dev(q.view(np.int16)), dev(codes), dev(scales), dev(topk), c_d, out, Qn, T, W,
                              swa_scale=s_d, swa_start=dev(start) if ring is not None else None,
                              swa_new=None if swa_new is None else dev(swa_new.view(np.int16)),
                              waves=waves, splits=splits)
        n = csa2.attn_workspace_size(args)
        csa2.sparse_attn(args, torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None)
        return host(out), host(c_d), host(s_d)

    ref_out, _, _ = run(full_c, full_s, None)
    got_out, got_c, got_s = run(stale_c, stale_s, new_bits)
    np.testing.assert_array_equal(got_out, ref_out)
    np.testing.assert_array_equal(got_c, full_c)
    np.testing.assert_array_equal(got_s, full_s)
    ref = oattn.sparse_attn(bf16_values(q), codes, scales, topk, swa8.swa_values(rc.reshape(-1, d), rs.reshape(-1))
                            .reshape(swa.shape), Qn, T, window=W)
    assert rownorm_err(got_out, ref) <= ATTN_TOL
