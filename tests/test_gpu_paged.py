"""GPU parity of the paged FP4 cache and the window ring buffer.

* csa2_quantize_kv_paged writes each new row's oracle codes and scales into
  the cache row its block table names (bit-exact), skips rows whose
  sequence, position or page is out of range, and leaves every other row
  untouched.
* csa2_sparse_attn over a paged cache (pages in shuffled order, spare and
  shared pages, -1 pages) gives bit-identical outputs to the same call over
  the contiguous cache, and matches the oracle within 2e-3.
* A window held as a ring (rows rotated by a per-sequence start slot) gives
  bit-identical outputs to the linear window, for bf16 and 8-bit rows.
Every attention case is also checked against the oracle within 2e-3."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from oracle import attention as oattn
from oracle import quant as oquant
from oracle import swa8 as oswa8
from tests.parity import ATTN_TOL, bf16_values, dev, host, rownorm_err
from tests.test_gpu_attn import make_case, oracle_out

pytestmark = pytest.mark.gpu


def oracle_out_8bit(q, codes, scales, topk, c8, s8, qn, T, W):
    """Oracle attention over a linear 8-bit window: E4M3 codes [B, R, d] with
    row scales [B, R], decoded by the oracle's own 8-bit window format."""
    d = c8.shape[-1]
    vals = oswa8.swa_values(c8.reshape(-1, d), s8.reshape(-1)).reshape(c8.shape)
    return oattn.sparse_attn(bf16_values(q), codes, scales, topk, vals, qn, T, window=W)


def page_layout(rng, B, T, P, spare=7):
    """A block table [B, max_pages] over a cache of n_phys pages in shuffled
    order (plus spare pages no sequence uses), and the cache row of every
    (sequence, position)."""
    max_pages = (T + P - 1) // P
    n_phys = B * max_pages + spare
    perm = rng.permutation(n_phys)[: B * max_pages].astype(np.int32)
    bt = perm.reshape(B, max_pages)
    t = np.arange(T)
    rows = bt[:, t // P] * P + t % P                     # [B, T]
    return bt, rows, n_phys * P


def paged_copy(codes, scales, rows, n_rows, fill=0x5A):
    """Scatter the contiguous cache rows (row b*T+t) to their paged rows."""
    B, T = rows.shape
    pc = np.full((n_rows, codes.shape[1]), fill, np.uint8)
    ps = np.full((n_rows, scales.shape[1]), 0x38, np.uint8)
    pc[rows.reshape(-1)] = codes[: B * T]
    ps[rows.reshape(-1)] = scales[: B * T]
    return pc, ps


def run_attn(q, codes, scales, topk, swa, qn, T, W, block_table=None, page_size=0, swa_scale=None, swa_start=None,
             kernel=0):
    nq, H, d = q.shape
    keep = [dev(q.view(np.int16)), dev(codes), dev(scales), dev(topk.astype(np.int32)),
            dev(swa.view(np.int16) if swa_scale is None else swa)]
    out = torch.full((nq, H, d), float("nan"), dtype=torch.float32, device="cuda")
    bt_d = dev(block_table.astype(np.int32)) if block_table is not None else None
    sc_d = dev(swa_scale.astype(np.float32)) if swa_scale is not None else None
    st_d = dev(np.asarray(swa_start, np.int32)) if swa_start is not None else None
    args = csa2.attn_args(keep[0], keep[1], keep[2], keep[3], keep[4], out, qn, T, W, swa_scale=sc_d,
                          block_table=bt_d, page_size=page_size, swa_start=st_d, kernel=kernel)
    n = csa2.attn_workspace_size(args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None
    csa2.sparse_attn(args, ws)
    return host(out)


PAGED_CASES = [  # (B, Qn, T, d, H, W, k, P)
    (2, 1, 1000, 512, 64, 128, 512, 64),
    (3, 1, 4099, 512, 64, 128, 512, 256),     # ragged last page
    (2, 3, 700, 128, 8, 128, 100, 16),
    (1, 6, 5000, 512, 64, 128, 512, 1),       # one row per page
    (4, 1, 300, 128, 16, 128, 512, 4096),     # one page holds a whole sequence
    (2, 1, 70000, 128, 8, 128, 512, 65536),   # the largest page size; two pages per sequence
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "B{}Q{}T{}d{}H{}P{}".format(*c[:5], c[7]))
def test_attn_paged_equals_contiguous(case):
    B, Qn, T, d, H, W, k, P = case
    codes, scales, q, swa, topk = make_case(sum(case), B, Qn, T, d, H, W, k)
    # a few positions past T and -1 slots stay empty on both paths
    topk[0, -3:] = [-1, T, T + 5]
    rng = np.random.default_rng(sum(case) + 1)
    bt, rows, n_rows = page_layout(rng, B, T, P)
    pc, ps = paged_copy(codes, scales, rows, n_rows)
    ref = run_attn(q, codes, scales, topk, swa, Qn, T, W)
    got = run_attn(q, pc, ps, topk, swa, Qn, T, W, block_table=bt, page_size=P)
    np.testing.assert_array_equal(got, ref)
    want = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert rownorm_err(got, want) <= ATTN_TOL


@pytest.mark.parametrize("P", [16, 256])
def test_attn_paged_with_8bit_window_ring(P):
    """All options together: paged FP4 cache, 8-bit window rows, window ring;
    bit-identical to the contiguous cache with a linear 8-bit window."""
    B, Qn, T, d, H, W, k = 3, 2, 3000, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(P + 3, B, Qn, T, d, H, W, k)
    R = swa.shape[1]
    c8, s8 = oswa8.quantize_swa_rows(bf16_values(swa).reshape(-1, d))
    c8, s8 = c8.reshape(B, R, d), s8.reshape(B, R).astype(np.float32)
    start = np.array([3, 0, R - 2], np.int32)
    ring = np.stack([np.roll(c8[b], start[b], axis=0) for b in range(B)])
    rsc = np.stack([np.roll(s8[b], start[b]) for b in range(B)])
    rng = np.random.default_rng(P)
    bt, rows, n_rows = page_layout(rng, B, T, P)
    pc, ps = paged_copy(codes, scales, rows, n_rows)
    ref = run_attn(q, codes, scales, topk, c8, Qn, T, W, swa_scale=s8)
    got = run_attn(q, pc, ps, topk, ring, Qn, T, W, block_table=bt, page_size=P, swa_scale=rsc, swa_start=start)
    np.testing.assert_array_equal(got, ref)
    want = oracle_out_8bit(q, codes, scales, topk, c8, s8, Qn, T, W)
    assert rownorm_err(got, want) <= ATTN_TOL


def test_attn_paged_shared_and_missing_pages():
    """Two sequences share their first pages (a common prefix); a page id of
    -1 or past the cache leaves its positions out, as -1 Top-K slots do."""
    B, Qn, T, d, H, W, k, P = 2, 1, 2048, 512, 64, 128, 512, 128
    codes, scales, q, swa, topk = make_case(5, B, Qn, T, d, H, W, k)
    codes[T:T + 4 * P] = codes[:4 * P]                    # sequence 1 starts with sequence 0's rows
    scales[T:T + 4 * P] = scales[:4 * P]
    rng = np.random.default_rng(6)
    bt, rows, n_rows = page_layout(rng, B, T, P)
    bt[1, :4] = bt[0, :4]                                 # shared physical pages
    rows = bt[:, np.arange(T) // P] * P + np.arange(T) % P
    pc, ps = paged_copy(codes, scales, rows, n_rows)
    bt[0, 7] = -1                                         # missing pages
    bt[1, 9] = n_rows // P + 3
    ref_topk = topk.copy()
    ref_topk[0][(topk[0] // P) == 7] = -1
    ref_topk[1][(topk[1] // P) == 9] = -1
    ref = run_attn(q, codes, scales, ref_topk, swa, Qn, T, W)
    got = run_attn(q, pc, ps, topk, swa, Qn, T, W, block_table=bt, page_size=P)
    np.testing.assert_array_equal(got, ref)
    # the oracle over the contiguous rows, with the missing pages' positions out
    want = oracle_out(q, codes, scales, ref_topk, swa, Qn, T, W)
    assert rownorm_err(got, want) <= ATTN_TOL


@pytest.mark.parametrize("swa8", [False, True])
def test_attn_window_ring_equals_linear(swa8):
    B, Qn, T, d, H, W, k = 3, 2, 1500, 512, 64, 128, 512
    codes, scales, q, swa, topk = make_case(11 + swa8, B, Qn, T, d, H, W, k)
    R = swa.shape[1]
    sc = None
    if swa8:
        c8, s8 = oswa8.quantize_swa_rows(bf16_values(swa).reshape(-1, d))
        swa, sc = c8.reshape(B, R, d), s8.reshape(B, R).astype(np.float32)
    start = np.array([0, 5, R - 1], np.int32)
    ring = np.empty_like(swa)
    rsc = None if sc is None else np.empty_like(sc)
    for b in range(B):
        ring[b] = np.roll(swa[b], start[b], axis=0)       # row r -> slot (r + start) % R
        if sc is not None:
            rsc[b] = np.roll(sc[b], start[b])
    ref = run_attn(q, codes, scales, topk, swa, Qn, T, W, swa_scale=sc)
    got = run_attn(q, codes, scales, topk, ring, Qn, T, W, swa_scale=rsc, swa_start=start)
    np.testing.assert_array_equal(got, ref)
    if swa8:
        want = oracle_out_8bit(q, codes, scales, topk, swa, sc, Qn, T, W)
    else:
        want = oracle_out(q, codes, scales, topk, swa, Qn, T, W)
    assert rownorm_err(got, want) <= ATTN_TOL


def test_quantize_kv_paged_matches_oracle():
    rng = np.random.default_rng(21)
    B, T, d, P = 4, 1000, 512, 64
    bt, rows, n_rows = page_layout(rng, B, T, P)
    n = 12
    x = rng.standard_normal((n, d)).astype(np.float32)
    seq = np.array([0, 1, 2, 3, 0, 1, 2, 3, 4, -1, 0, 3], np.int32)      # 4 and -1: no such sequence
    pos = np.array([999, 0, 63, 64, 500, 998, 1, 640, 5, 5, T + 100, -2], np.int32)   # T + 100 > 16 pages
    bt_used = bt.copy()
    bt_used[2, 0] = -1                                    # rows 2 and 6 (sequence 2, page 0): no page
    codes = torch.full((n_rows, d // 2), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_rows, d // 16), 0xA5, dtype=torch.uint8, device="cuda")
    csa2.quantize_kv_paged(dev(x), dev(seq), dev(pos), dev(bt_used), P, codes, scales)
    got_c, got_s = host(codes), host(scales)
    rc, rs = oquant.quantize_rows(x)
    written = np.zeros(n_rows, bool)
    for r in range(n):
        b, t = int(seq[r]), int(pos[r])
        if not (0 <= b < B and 0 <= t < bt.shape[1] * P) or bt_used[b, t // P] < 0:
            continue
        row = int(bt_used[b, t // P]) * P + t % P
        np.testing.assert_array_equal(got_c[row], rc[r])
        np.testing.assert_array_equal(got_s[row], rs[r])
        written[row] = True
    assert written.sum() == 6
    assert np.all(got_c[~written] == 0xA5) and np.all(got_s[~written] == 0xA5)


@pytest.mark.parametrize("rows,split", [(32, False), (32, True), (600, False)])
def test_index_append_paged_equals_separate_calls(rows, split):
    """csa2_index_full_append_paged (and the split select form) give the same
    pool, Top-512 and paged cache rows as csa2_index_full followed by
    csa2_quantize_kv_paged; 600 rows x 32 groups exceed the extra-workgroup
    job and take a launch of their own."""
    rng = np.random.default_rng(rows + split)
    B, T, d, P, HI, DI = 4, 5000, 512, 64, 8, 128
    iq = rng.integers(-8, 9, size=(B, HI, DI), dtype=np.int8)
    iw = rng.integers(1, 9, size=(B, HI)).astype(np.float32)
    ik = rng.integers(-8, 9, size=(B, T, DI), dtype=np.int8)
    bt, _, n_rows = page_layout(rng, B, T, P)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    seq = rng.integers(0, B, size=rows).astype(np.int32)
    pos = rng.permutation(T)[:rows].astype(np.int32)              # distinct positions -> distinct rows
    d_in = [dev(a) for a in (iq, iw, ik, x, seq, pos, bt)]
    args = csa2.index_args(d_in[0], d_in[1], d_in[2], 1)
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    outs = []
    for fused in (True, False):
        pool = torch.full((B, 2048), -7, dtype=torch.int32, device="cuda")
        topk = torch.full((B, 512), -7, dtype=torch.int32, device="cuda")
        codes = torch.full((n_rows, d // 2), 0xA5, dtype=torch.uint8, device="cuda")
        scales = torch.full((n_rows, d // 16), 0xA5, dtype=torch.uint8, device="cuda")
        pg = (d_in[3], d_in[4], d_in[5], d_in[6], P, codes, scales)
        if fused and split:
            csa2.index_scan(args, ws)
            csa2.index_select_append_paged(args, pool, topk, ws, *pg)
        elif fused:
            csa2.index_full_append_paged(args, pool, topk, ws, *pg)
        else:
            csa2.index_full(args, pool, topk, ws)
            csa2.quantize_kv_paged(d_in[3], d_in[4], d_in[5], d_in[6], P, codes, scales)
        outs.append([host(pool), host(topk), host(codes), host(scales)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    rc, rs = oquant.quantize_rows(x)
    dst = bt[seq, pos // P].astype(np.int64) * P + pos % P
    np.testing.assert_array_equal(outs[0][2][dst], rc)
    np.testing.assert_array_equal(outs[0][3][dst], rs)


@pytest.mark.parametrize("split", [(0, 0), (4, 1), (8, 3)], ids=["auto", "w4s1", "w8s3"])
def test_attn_paged_rows_out_and_rows_in(split):
    """A paged call with topk_rows_out writes every Top-K slot's cache row
    (-1 for empty slots, positions past T and missing pages); a call given
    those rows (topk_is_rows, no block table) is bit-identical to the paged
    call, and both match the oracle."""
    waves, splits = split
    B, Qn, T, d, H, W, k, P = 3, 2, 3000, 512, 64, 128, 512, 64
    codes, scales, q, swa, topk = make_case(41, B, Qn, T, d, H, W, k)
    topk[0, -3:] = [-1, T, T + 5]
    rng = np.random.default_rng(42)
    bt, rows, n_rows = page_layout(rng, B, T, P)
    pc, ps = paged_copy(codes, scales, rows, n_rows)
    bt[2, 5] = -1                                         # a missing page
    want_rows = np.full((B * Qn, k), -1, np.int32)
    for i in range(B * Qn):
        b = i // Qn
        for s, t in enumerate(topk[i]):
            if 0 <= t < T and bt[b, t // P] >= 0:
                want_rows[i, s] = bt[b, t // P] * P + t % P
    q_d, c_d, s_d, sw_d = dev(q.view(np.int16)), dev(pc), dev(ps), dev(swa.view(np.int16))

    def run(tk, **kw):
        out = torch.full((B * Qn, H, d), float("nan"), dtype=torch.float32, device="cuda")
        args = csa2.attn_args(q_d, c_d, s_d, tk, sw_d, out, Qn, T, W, waves=waves, splits=splits, **kw)
        n = csa2.attn_workspace_size(args)
        csa2.sparse_attn(args, torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") if n else None)
        return host(out)

    rows_d = torch.full((B * Qn, k), -7, dtype=torch.int32, device="cuda")
    paged = run(dev(topk), block_table=dev(bt), page_size=P, topk_rows_out=rows_d)
    np.testing.assert_array_equal(host(rows_d), want_rows)
    plain = run(dev(topk), block_table=dev(bt), page_size=P)
    np.testing.assert_array_equal(paged, plain)
    from_rows = run(rows_d, topk_is_rows=True)
    np.testing.assert_array_equal(from_rows, paged)
    ref_topk = topk.copy()
    ref_topk[4:6][(topk[4:6] // P) == 5] = -1             # sequence 2's missing page
    want = oracle_out(q, codes, scales, ref_topk, swa, Qn, T, W)
    assert rownorm_err(paged, want) <= ATTN_TOL
