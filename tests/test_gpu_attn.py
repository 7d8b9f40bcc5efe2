"""GPU parity of csa2_sparse_attn against the FP64 oracle (row-normalised
error <= 2e-3), on small ragged shapes covering the edge cases and on the
T=4096 single-sequence and batch-32 / 64K-entry decode workloads."""
import math

import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from fp4_kv_cache_e4m3_amd import synth
from oracle import attention as oattn
from oracle import indexer as oidx
from oracle import quant as oquant
from tests.parity import ATTN_TOL, bf16_values, dev, host, oracle_attention, rownorm_err

pytestmark = pytest.mark.gpu


def gpu_attn(q_bits, codes, scales, topk, swa_bits, qn, T, window, swa_len=None, sm_scale=0.0, waves=0, splits=0,
             kernel=0):
    nq, H, d = q_bits.shape
    q_d = dev(q_bits.view(np.int16))
    c_d, s_d = dev(codes), dev(scales)
    t_d = dev(topk.astype(np.int32)) if topk is not None and topk.shape[1] > 0 else None
    sw_d = dev(swa_bits.view(np.int16)) if window > 0 else None
    sl_d = dev(np.asarray(swa_len, np.int32)) if swa_len is not None else None
    out = torch.full((nq, H, d), float("nan"), dtype=torch.float32, device="cuda")
    args = csa2.attn_args(q_d, c_d, s_d, t_d, sw_d, out, qn, T, window, sl_d, sm_scale, waves=waves, splits=splits,
                          kernel=kernel)
    if t_d is None:
        args.topk_k = 0
    n = csa2.attn_workspace_size(args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None
    csa2.sparse_attn(args, ws)
    return host(out)


def make_case(seed, B, Qn, T, d, H, W, k, fill=0.8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B * T, d)).astype(np.float32) if T else np.zeros((1, d), np.float32)
    codes, scales = oquant.quantize_rows(x)
    q = synth.f32_to_bf16_bits(rng.standard_normal((B * Qn, H, d)).astype(np.float32))
    swa = synth.f32_to_bf16_bits(rng.standard_normal((B, max(W - 1 + Qn, 1), d)).astype(np.float32))
    topk = np.full((B * Qn, k), -1, dtype=np.int32)
    for i in range(B * Qn):
        n = min(T, int(rng.integers(0, k + 1) if fill is None else int(k * fill)))
        if n:
            topk[i, :n] = np.sort(rng.choice(T, size=n, replace=False))
    return codes, scales, q, swa, topk


def oracle_out(q, codes, scales, topk, swa, qn, T, W, swa_len=None, sm_scale=None):
    return oattn.sparse_attn(bf16_values(q), codes, scales, topk, bf16_values(swa), qn, T, window=W,
                             sm_scale=sm_scale, swa_len=swa_len)


CASES = [  # (B, Qn, T, d, H, W, k)
    (1, 1, 300, 128, 8, 128, 512),      # Top-K longer than the context: trailing -1
    (2, 1, 1000, 512, 64, 128, 512),
    (2, 3, 700, 512, 16, 128, 100),     # ragged k, causal window over 3 queries
    (1, 6, 5000, 512, 64, 128, 512),    # 1 + 5 draft queries
    (3, 1, 50, 128, 24, 37, 40),        # heads not a multiple of 16, odd window
    (2, 2, 64, 128, 8, 0, 64),          # no window at all
    (1, 1, 0, 128, 8, 128, 512),        # empty main cache: window only
    (4, 1, 2000, 512, 128, 128, 512),   # 128 heads
    (1, 1, 6000, 512, 32, 128, 2048),   # longest Top-K row: many FP4 tile pairs per wave
    (2, 2, 3000, 512, 16, 64, 1000),    # odd number of FP4 tiles, shorter window
    (1, 3, 900, 128, 16, 128, 17),      # one full FP4 tile and a one-entry tail
    (1, 2, 3000, 512, 16, 1024, 512),   # the longest window the header allows (64 window tiles)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}Q{}T{}d{}H{}W{}k{}".format(*c))
def test_attn_matches_oracle(case):
    B, Qn, T, d, H, W, k = case
    codes, scales, q, swa, topk = make_case(sum(case), B, Qn, T, d, H, W, k, fill=None)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    err = rownorm_err(got, ref)
    assert err <= ATTN_TOL, err


def test_attn_empty_and_partial_window():
    B, Qn, T, d, H, W, k = 3, 2, 400, 512, 16, 128, 512
    codes, scales, q, swa, topk = make_case(5, B, Qn, T, d, H, W, k)
    topk[1] = -1                                   # query 1: window only
    swa_len = np.array([129, 5, 0], np.int32)      # seq 2: no valid window row
    topk[4:6] = -1                                 # seq 2 queries have nothing at all
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, swa_len=swa_len)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W, swa_len=swa_len)
    assert np.all(got[4:6] == 0.0)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_out_of_range_positions_are_ignored():
    B, Qn, T, d, H, W, k = 2, 1, 100, 128, 8, 16, 64
    codes, scales, q, swa, topk = make_case(6, B, Qn, T, d, H, W, k, fill=0.5)
    bad = topk.copy()
    bad[:, 40] = T + 5                             # beyond the sequence
    bad[:, 41] = -3
    got = gpu_attn(q, codes, scales, bad, swa, Qn, T, W)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_custom_scale_and_dominant_entry():
    B, Qn, T, d, H, W, k = 1, 1, 200, 512, 16, 16, 32
    codes, scales, q, swa, topk = make_case(7, B, Qn, T, d, H, W, k)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, sm_scale=0.3)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W, sm_scale=0.3)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_deterministic():
    case = (2, 1, 1000, 512, 64, 128, 512)
    codes, scales, q, swa, topk = make_case(8, *case)
    a = gpu_attn(q, codes, scales, topk, swa, 1, 1000, 128)
    b = gpu_attn(q, codes, scales, topk, swa, 1, 1000, 128)
    assert np.array_equal(a, b)


def test_attn_single_sequence_t4096():
    w = synth.C1
    iq, iw, ik = synth.index_q(w), synth.index_w(w), synth.index_k_all(w)
    _, topk = oidx.index_full(iq, iw, ik, 1)
    x = synth.kv_source(w, 0)
    codes, scales = oquant.quantize_rows(x)
    q, swa = synth.attn_q_bf16(w), synth.swa_bf16(w)
    got = gpu_attn(q, codes, scales, topk, swa, 1, w.kv_len, w.window)
    ref = oracle_attention(w, q, swa, topk, with_new_rows=False)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_batch32_t65536_layer():
    w = synth.C2
    # Top-512 from the oracle's own indexer; the KV rows from the oracle's quantiser
    iq, iw, ik = synth.index_q(w), synth.index_w(w), synth.index_k_all(w)
    _, topk = oidx.index_full(iq, iw, ik, 1)
    del ik
    q, swa = synth.attn_q_bf16(w, 2), synth.swa_bf16(w, 2)
    # stage the selected rows (plus nothing else) into a compact cache: position p of
    # sequence b -> row b*T + p of a cache that is zero except at selected rows
    T = w.kv_len
    codes = np.zeros((w.batch * T, w.dim // 2), np.uint8)
    scales = np.zeros((w.batch * T, w.dim // 16), np.uint8)
    from tests.parity import oracle_kv_rows
    for b in range(w.batch):
        pos = topk[b][topk[b] >= 0]
        c, s = oracle_kv_rows(w, b, pos, with_new_rows=False)
        codes[b * T + pos] = c
        scales[b * T + pos] = s
    got = gpu_attn(q, codes, scales, topk, swa, 1, T, w.window)
    ref = oracle_attention(w, q, swa, topk, with_new_rows=False)
    err = rownorm_err(got, ref)
    assert err <= ATTN_TOL, err


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("splits", [1, 2, 3, 4, 40])
def test_attn_work_split_sweep(waves, splits):
    """Every work split the caller may choose (waves per workgroup x splits of
    the tile list, the latter merged by the second kernel; 40 splits = one
    16-entry tile each) stays within 2e-3
    of the oracle at the decode layer's shape (512 Top-K + 128-row window, 64
    heads, d = 512), and each split is bit-identical from run to run."""
    B, Qn, T, d, H, W, k = 8, 1, 8000, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(31, B, Qn, T, d, H, W, k, fill=1.0)
    a = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, waves=waves, splits=splits)
    b = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, waves=waves, splits=splits)
    assert np.array_equal(a, b)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    err = rownorm_err(a, ref)
    assert err <= ATTN_TOL, err


def test_attn_large_q_magnitudes():
    """|Q| up to about 4e4 (inside the documented fp16 range of the QK^T
    operands): Q is scaled by 2^13 and the FP4 rows and window by 2^-13, so
    the logits keep their N(0,1) spread and the softmax stays well
    conditioned."""
    B, Qn, T, d, H, W, k = 2, 1, 3000, 512, 64, 128, 512
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((B * T, d)) * 2.0 ** -13).astype(np.float32)
    codes, scales = oquant.quantize_rows(x)
    q = synth.f32_to_bf16_bits((rng.standard_normal((B * Qn, H, d)) * 2.0 ** 13).astype(np.float32))
    swa = synth.f32_to_bf16_bits((rng.standard_normal((B, W - 1 + Qn, d)) * 2.0 ** -13).astype(np.float32))
    assert np.abs(bf16_values(q)).max() > 2.0 ** 15
    topk = np.stack([np.sort(rng.choice(T, size=k, replace=False)) for _ in range(B * Qn)]).astype(np.int32)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_large_window_values_and_tiny_q():
    """Window values up to about 4e4 (they are V in fp16 for PV) against a Q
    scaled by 2^-13, whose smaller elements fall below fp16's normal range
    (the documented 2^-25 absolute conversion loss)."""
    B, Qn, T, d, H, W, k = 2, 2, 3000, 512, 32, 128, 512
    codes, scales, q, swa, topk = make_case(43, B, Qn, T, d, H, W, k, fill=1.0)
    q = synth.f32_to_bf16_bits((bf16_values(q) * 2.0 ** -13).astype(np.float32))
    swa = synth.f32_to_bf16_bits((bf16_values(swa) * 2.0 ** 13).astype(np.float32))
    assert np.abs(bf16_values(swa)).max() > 2.0 ** 15
    assert (np.abs(bf16_values(q)) < 2.0 ** -14).mean() > 0.2
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL


@pytest.mark.parametrize("kernel", [1, 2])
def test_attn_rows_at_the_top_of_the_offset_range(kernel):
    """Top-K rows at both ends of a cache whose byte size comes within 8 KiB
    of 4 GiB (T * codes_stride < 4 GiB - 8 KiB, the header's bound): the
    32-bit row offsets of the last rows and the out-of-range offset that
    empty slots read stay apart.  The oracle sees the 512 selected rows as a
    512-row cache."""
    d, H, W, k, Qn = 512, 64, 128, 512, 1
    T = ((4 << 30) - (8 << 10)) // (d // 2) - 1              # the largest T under the bound
    codes_s, scales_s, q, swa, _ = make_case(77, 1, Qn, k, d, H, W, k)
    rng = np.random.default_rng(78)
    ends = np.array([0, 1, T // 2, T - 2, T - 1], np.int64)
    mid = rng.choice(np.arange(2, T - 2, 7919, dtype=np.int64), size=k - len(ends) - 1, replace=False)
    pos = np.sort(np.concatenate([ends, mid]))                 # 511 rows and one empty slot
    codes = torch.zeros((T, d // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((T, d // 16), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(pos).cuda()
    codes[idx] = dev(codes_s[:len(pos)])
    scales[idx] = dev(scales_s[:len(pos)])
    topk = np.full((1, k), -1, np.int32)
    topk[0, :len(pos)] = pos
    out = torch.full((1, H, d), float("nan"), dtype=torch.float32, device="cuda")
    args = csa2.attn_args(dev(q.view(np.int16)), codes, scales, dev(topk), dev(swa.view(np.int16)), out, Qn, T, W,
                          kernel=kernel)
    n = csa2.attn_workspace_size(args)
    csa2.sparse_attn(args, torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None)
    got = host(out)
    small = np.full((1, k), -1, np.int32)
    small[0, :len(pos)] = np.arange(len(pos), dtype=np.int32)
    ref = oracle_out(q, codes_s, scales_s, small, swa, Qn, k, W)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL
    del codes, scales
    torch.cuda.empty_cache()
