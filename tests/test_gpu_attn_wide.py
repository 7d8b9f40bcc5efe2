"""GPU parity of the one-workgroup-per-query attention kernel (kernel = 2,
the library's choice for prefill-sized calls) against the FP64 oracle
(row-normalised error <= 2e-3): ragged Top-K rows and windows, partial and
several 64-head groups, empty inputs, paged caches and window rings, the
documented magnitude range, and a 600-query chunk where the library picks
the kernel by itself."""
import numpy as np
import pytest

from fp4_kv_cache_e4m3_amd import synth
from oracle import quant as oquant
from tests.parity import ATTN_TOL, bf16_values, rownorm_err
from tests.test_gpu_attn import gpu_attn, make_case, oracle_out
from tests.test_gpu_paged import page_layout, paged_copy, run_attn

pytestmark = pytest.mark.gpu

WIDE_CASES = [  # (B, Qn, T, d, H, W, k)
    (2, 1, 1000, 512, 64, 128, 512),
    (2, 3, 700, 512, 16, 128, 100),     # 16 heads: a partial 64-head group; ragged k
    (1, 6, 5000, 512, 64, 128, 512),
    (4, 1, 2000, 512, 128, 128, 512),   # two head groups
    (3, 2, 900, 512, 72, 128, 300),     # the second group holds 8 heads
    (1, 1, 6000, 512, 32, 128, 2048),   # longest Top-K row (64 FP4 tiles)
    (2, 2, 3000, 512, 16, 64, 1000),    # odd number of FP4 tiles, shorter window
    (1, 2, 500, 512, 64, 100, 33),      # one full FP4 tile and a one-entry tail; window not a tile multiple
    (2, 2, 64, 512, 8, 0, 64),          # no window at all
    (1, 1, 0, 512, 8, 128, 512),        # empty main cache: window only
    (1, 3, 900, 512, 64, 1, 17),        # one-row window
    (1, 2, 3000, 512, 64, 1024, 512),   # the longest window the header allows (32 window tiles)
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "B{}Q{}T{}d{}H{}W{}k{}".format(*c))
def test_attn_wide_matches_oracle(case):
    B, Qn, T, d, H, W, k = case
    codes, scales, q, swa, topk = make_case(sum(case) + 100, B, Qn, T, d, H, W, k, fill=None)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, kernel=2)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    err = rownorm_err(got, ref)
    assert err <= ATTN_TOL, err


def test_attn_wide_empty_and_partial_window():
    B, Qn, T, d, H, W, k = 3, 2, 400, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(5, B, Qn, T, d, H, W, k)
    topk[1] = -1                                   # query 1: window only
    swa_len = np.array([129, 5, 0], np.int32)      # seq 2: no valid window row
    topk[4:6] = -1                                 # seq 2 queries have nothing at all
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, swa_len=swa_len, kernel=2)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W, swa_len=swa_len)
    assert np.all(got[4:6] == 0.0)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_wide_out_of_range_positions_and_custom_scale():
    B, Qn, T, d, H, W, k = 2, 1, 100, 512, 64, 16, 64
    codes, scales, q, swa, topk = make_case(6, B, Qn, T, d, H, W, k, fill=0.5)
    bad = topk.copy()
    bad[:, 40] = T + 5                             # beyond the sequence
    bad[:, 41] = -3
    got = gpu_attn(q, codes, scales, bad, swa, Qn, T, W, sm_scale=0.3, kernel=2)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W, sm_scale=0.3)
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_wide_deterministic_and_close_to_head_group_kernel():
    case = (2, 1, 1000, 512, 64, 128, 512)
    codes, scales, q, swa, topk = make_case(8, *case)
    a = gpu_attn(q, codes, scales, topk, swa, 1, 1000, 128, kernel=2)
    b = gpu_attn(q, codes, scales, topk, swa, 1, 1000, 128, kernel=2)
    assert np.array_equal(a, b)
    c = gpu_attn(q, codes, scales, topk, swa, 1, 1000, 128, kernel=1)
    ref = oracle_out(q, codes, scales, topk, swa, 1, 1000, 128)
    assert rownorm_err(a, ref) <= ATTN_TOL and rownorm_err(c, ref) <= ATTN_TOL


def test_attn_wide_large_q_magnitudes():
    """|Q| up to about 4e4 against FP4 rows and window scaled by 2^-13 (the
    fp16 range of the QK^T operands)."""
    B, Qn, T, d, H, W, k = 2, 1, 3000, 512, 64, 128, 512
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((B * T, d)) * 2.0 ** -13).astype(np.float32)
    codes, scales = oquant.quantize_rows(x)
    q = synth.f32_to_bf16_bits((rng.standard_normal((B * Qn, H, d)) * 2.0 ** 13).astype(np.float32))
    swa = synth.f32_to_bf16_bits((rng.standard_normal((B, W - 1 + Qn, d)) * 2.0 ** -13).astype(np.float32))
    assert np.abs(bf16_values(q)).max() > 2.0 ** 15
    topk = np.stack([np.sort(rng.choice(T, size=k, replace=False)) for _ in range(B * Qn)]).astype(np.int32)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, kernel=2)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL


def test_attn_wide_large_window_values_and_tiny_q():
    B, Qn, T, d, H, W, k = 2, 2, 3000, 512, 32, 128, 512
    codes, scales, q, swa, topk = make_case(43, B, Qn, T, d, H, W, k, fill=1.0)
    q = synth.f32_to_bf16_bits((bf16_values(q) * 2.0 ** -13).astype(np.float32))
    swa = synth.f32_to_bf16_bits((bf16_values(swa) * 2.0 ** 13).astype(np.float32))
    assert np.abs(bf16_values(swa)).max() > 2.0 ** 15
    assert (np.abs(bf16_values(q)) < 2.0 ** -14).mean() > 0.2
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, kernel=2)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert np.all(np.isfinite(got))
    assert rownorm_err(got, ref) <= ATTN_TOL


@pytest.mark.parametrize("P", [1, 64])
def test_attn_wide_paged_and_ring(P):
    """Paged cache (shuffled pages) and a window ring: bit-identical to the
    contiguous cache with a linear window, and within 2e-3 of the oracle."""
    B, Qn, T, d, H, W, k = 3, 2, 2000, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(P + 17, B, Qn, T, d, H, W, k)
    topk[0, -3:] = [-1, T, T + 5]
    rng = np.random.default_rng(P)
    bt, rows, n_rows = page_layout(rng, B, T, P)
    pc, ps = paged_copy(codes, scales, rows, n_rows)
    R = swa.shape[1]
    start = np.array([0, 5, R - 1], np.int32)
    ring = np.stack([np.roll(swa[b], start[b], axis=0) for b in range(B)])
    ref = run_attn(q, codes, scales, topk, swa, Qn, T, W, kernel=2)
    got = run_attn(q, pc, ps, topk, ring, Qn, T, W, block_table=bt, page_size=P, swa_start=start, kernel=2)
    np.testing.assert_array_equal(got, ref)
    want = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert rownorm_err(got, want) <= ATTN_TOL


def test_attn_prefill_chunk_library_choice():
    """600 query tokens of one sequence (a prefill chunk, causal window over
    the chunk): the library picks the one-workgroup-per-query kernel by
    itself; every query is checked against the oracle."""
    B, Qn, T, d, H, W, k = 1, 600, 4000, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(77, B, Qn, T, d, H, W, k, fill=1.0)
    got = gpu_attn(q, codes, scales, topk, swa, Qn, T, W)
    same = gpu_attn(q, codes, scales, topk, swa, Qn, T, W, kernel=2)
    np.testing.assert_array_equal(got, same)
    ref = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert rownorm_err(got, ref) <= ATTN_TOL
