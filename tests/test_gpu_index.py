"""GPU parity of csa2_index_full / csa2_index_reindex against the oracle:
bit-exact pools and Top-512 lists (including the -1 padding), at small ragged
shapes, at the single-sequence T=4096 workload and at the full batch-32,
64K-entry decode workload."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from fp4_kv_cache_e4m3_amd import synth
from oracle import indexer as oidx
from tests.parity import dev, host

pytestmark = pytest.mark.gpu


def run_full(iq, iw, ik, qn, n_visible=None, with_pool=True):
    iq_d, iw_d, ik_d = dev(iq), dev(iw), dev(ik)
    nv_d = dev(np.asarray(n_visible, dtype=np.int32)) if n_visible is not None else None
    nq = iq.shape[0]
    pool = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
    args = csa2.index_args(iq_d, iw_d, ik_d, qn, nv_d)
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    csa2.index_full(args, pool if with_pool else None, topk, ws)
    return host(pool), host(topk)


def run_reindex(iq, iw, ik, qn, pool, n_visible=None):
    iq_d, iw_d, ik_d = dev(iq), dev(iw), dev(ik)
    nv_d = dev(np.asarray(n_visible, dtype=np.int32)) if n_visible is not None else None
    topk = torch.full((iq.shape[0], 512), -7, dtype=torch.int32, device="cuda")
    args = csa2.index_args(iq_d, iw_d, ik_d, qn, nv_d)
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    csa2.index_reindex(args, dev(pool.astype(np.int32)), topk, ws)
    return host(topk)


def inputs(seed, B, Qn, T, HI, DI, r, wmax):
    rng = np.random.default_rng(seed)
    iq = rng.integers(-r, r + 1, size=(B * Qn, HI, DI), dtype=np.int8)
    iw = rng.integers(1, wmax + 1, size=(B * Qn, HI)).astype(np.float32)
    ik = rng.integers(-r, r + 1, size=(B, T, DI), dtype=np.int8)
    return iq, iw, ik


CASES = [  # (B, Qn, T, H_I, D_I, r, wmax)
    (1, 1, 1, 2, 64, 4, 4),
    (2, 1, 9, 2, 64, 4, 4),
    (1, 1, 4096, 2, 64, 4, 4),
    (3, 1, 5003, 8, 128, 8, 8),
    (2, 6, 20011, 8, 128, 8, 8),      # several queries per sequence, pool drops blocks
    (2, 4, 17003, 16, 64, 2, 2),
    (2, 3, 16400, 4, 128, 1, 1),      # heavy ties
    (1, 5, 300, 2, 64, 1, 3),
    (2, 1, 33000, 8, 64, 0, 1),       # all scores equal
    (1, 2, 100003, 8, 128, 8, 8),     # more than 8,192 blocks: super-block pre-selection
    (1, 3, 300001, 8, 64, 1, 2),      # ... with heavy ties
    (1, 1, 262144, 2, 64, 0, 1),      # ... all scores equal
    (1, 1, 8192, 2, 64, 0, 1),        # all equal, 1,024 blocks: every block a Top-512 candidate
    (1, 1, 8200, 2, 64, 0, 1),        # all equal, 1,025 candidate blocks: the pool is searched
    (2, 1, 12000, 2, 64, 1, 1),       # ties spread over the candidate threshold
    (1, 2, 4000, 2, 64, 1, 2),        # fewer than 512 blocks, more than 512 positions
    (2, 1, 2500, 8, 128, 8, 8),       # ... without heavy ties
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}Q{}T{}H{}D{}".format(*c[:5]))
def test_index_full_matches_oracle(case):
    B, Qn, T, HI, DI, r, wmax = case
    iq, iw, ik = inputs(hash(case) % 1000, B, Qn, T, HI, DI, r, wmax)
    pool, topk = run_full(iq, iw, ik, Qn)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)


def test_index_full_n_visible_ragged():
    B, Qn, T = 3, 4, 21000
    iq, iw, ik = inputs(11, B, Qn, T, 8, 128, 3, 5)
    nv = np.array([T, 0, 1, 7, 8, 9, 16, 17, 513, 16385, 20999, 12345], dtype=np.int32)
    pool, topk = run_full(iq, iw, ik, Qn, nv)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn, nv)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)


def test_index_full_n_visible_ragged_large():
    B, Qn, T = 1, 6, 150001
    iq, iw, ik = inputs(12, B, Qn, T, 8, 128, 2, 3)
    nv = np.array([T, 65537, 65535, 131073, 8, 149999], dtype=np.int32)
    pool, topk = run_full(iq, iw, ik, Qn, nv)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn, nv)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)


def test_index_full_without_pool_output():
    iq, iw, ik = inputs(3, 2, 1, 3000, 8, 128, 8, 8)
    _, topk = run_full(iq, iw, ik, 1, with_pool=False)
    _, rtopk = oidx.index_full(iq, iw, ik, 1)
    np.testing.assert_array_equal(topk, rtopk)


def test_index_full_single_sequence_t4096():
    w = synth.C1
    iq, iw, ik = synth.index_q(w), synth.index_w(w), synth.index_k_all(w)
    pool, topk = run_full(iq, iw, ik, 1)
    rpool, rtopk = oidx.index_full(iq, iw, ik, 1)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)


@pytest.fixture(scope="module")
def c2_inputs():
    w = synth.C2
    return w, synth.index_q(w), synth.index_w(w), synth.index_k_all(w)


def test_index_full_batch32_t65536(c2_inputs):
    w, iq, iw, ik = c2_inputs
    pool, topk = run_full(iq, iw, ik, 1)
    rpool, rtopk = oidx.index_full(iq, iw, ik, 1)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)
    # repeat: bit-identical
    pool2, topk2 = run_full(iq, iw, ik, 1)
    np.testing.assert_array_equal(pool, pool2)
    np.testing.assert_array_equal(topk, topk2)


def test_index_reindex_batch32_t65536(c2_inputs):
    w, _, _, ik = c2_inputs
    iq0, iw0 = synth.index_q(w, 0, pool_source=True), synth.index_w(w, 0, pool_source=True)
    rpool, rtopk0 = oidx.index_full(iq0, iw0, ik, 1)
    iq, iw = synth.index_q(w, 1), synth.index_w(w, 1)
    topk = run_reindex(iq, iw, ik, 1, rpool)
    np.testing.assert_array_equal(topk, oidx.index_reindex(iq, iw, ik, 1, rpool))
    # invariant: rescoring with the Full layer's own q reproduces its Top-512
    np.testing.assert_array_equal(run_reindex(iq0, iw0, ik, 1, rpool), rtopk0)


# Reindex cases: ragged shapes, heavy ties, all-equal scores (every pool block
# a candidate: the 16,384-position select), 1,024 candidate blocks exactly
REINDEX_CASES = CASES[3:7] + [(2, 1, 33000, 8, 64, 0, 1), (1, 1, 8192, 2, 64, 0, 1), (2, 1, 12000, 2, 64, 1, 1)]


@pytest.mark.parametrize("case", REINDEX_CASES, ids=lambda c: "B{}Q{}T{}H{}D{}r{}".format(*c[:6]))
def test_index_reindex_matches_oracle(case):
    B, Qn, T, HI, DI, r, wmax = case
    iq, iw, ik = inputs(hash(case) % 997, B, Qn, T, HI, DI, r, wmax)
    rpool, _ = oidx.index_full(iq, iw, ik, Qn)
    iq2, iw2, _ = inputs(hash(case) % 991 + 1, B, Qn, T, HI, DI, r, wmax)
    nv = np.full(B * Qn, T, dtype=np.int32)
    nv[0] = T // 2
    topk = run_reindex(iq2, iw2, ik, Qn, rpool, nv)
    np.testing.assert_array_equal(topk, oidx.index_reindex(iq2, iw2, ik, Qn, rpool, nv))


# From 2^19 positions on, the scan writes only block maxima and the Top-512 is
# taken from the pool rescored with the layer's own query.
LONG_CASES = [  # (B, Qn, T, H_I, D_I, r, wmax)
    (1, 2, 1 << 19, 8, 64, 1, 2),           # at the threshold, heavy ties
    (1, 1, (1 << 19) + 3, 2, 64, 0, 1),     # all scores equal, ragged tail
    (2, 3, 600001, 8, 128, 8, 8),
    (1, 2, 700000, 16, 64, 2, 2),
    (1, 2, 530000, 4, 128, 1, 1),
]


@pytest.mark.parametrize("case", LONG_CASES, ids=lambda c: "B{}Q{}T{}H{}D{}".format(*c[:5]))
def test_index_full_long_matches_oracle(case):
    B, Qn, T, HI, DI, r, wmax = case
    iq, iw, ik = inputs(hash(case) % 1000, B, Qn, T, HI, DI, r, wmax)
    pool, topk = run_full(iq, iw, ik, Qn)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)
    _, topk2 = run_full(iq, iw, ik, Qn, with_pool=False)      # the pool then lives in the workspace
    np.testing.assert_array_equal(topk2, rtopk)


def test_index_full_long_n_visible_ragged():
    B, Qn, T = 1, 8, (1 << 19) + 5
    iq, iw, ik = inputs(13, B, Qn, T, 8, 128, 3, 5)
    nv = np.array([T, 0, 1, 9, 513, 65537, 300001, T - 1], dtype=np.int32)
    pool, topk = run_full(iq, iw, ik, Qn, nv)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn, nv)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)
    assert np.all(pool[1] == -1) and np.all(topk[1] == -1)


def test_index_full_verify_1m_entries():
    """1,048,576 entries per sequence, 1 + 5 draft queries per sequence: the
    131,072-block pool select that streams its block keys from memory.  The
    oracle checks the first and the last sequence (12 of the 48 queries)."""
    w = synth.C5
    iq, iw = synth.index_q(w), synth.index_w(w)
    ik = synth.index_k_all(w)
    pool, topk = run_full(iq, iw, ik, w.q_per_seq)
    for b in (0, w.batch - 1):
        sl = slice(b * w.q_per_seq, (b + 1) * w.q_per_seq)
        rpool, rtopk = oidx.index_full(iq[sl], iw[sl], ik[b:b + 1], w.q_per_seq)
        np.testing.assert_array_equal(pool[sl], rpool)
        np.testing.assert_array_equal(topk[sl], rtopk)


@pytest.mark.parametrize("rows,dim,split", [(32, 512, False), (32, 512, True), (300, 512, False), (7, 128, True)],
                         ids=["32x512", "32x512-split", "300x512-own-launch", "7x128-split"])
def test_index_append_matches_oracle(rows, dim, split):
    """csa2_index_full_append / csa2_index_select_append: the Full indexer and
    the FP4 quantisation of new main-KV rows in one call (small jobs ride in
    the selection launch, 300 x 512 = 9,600 groups takes its own launch);
    pool, Top-512, codes and scales bit-exact against the oracle, and rows of
    the cache outside the job untouched."""
    from oracle import quant as oquant
    B, Qn, T = 3, 1, 5003
    iq, iw, ik = inputs(77, B, Qn, T, 8, 128, 8, 8)
    x = np.random.default_rng(78).standard_normal((rows, dim), dtype=np.float32)
    rpool, rtopk = oidx.index_full(iq, iw, ik, Qn)
    rc, rs = oquant.quantize_rows(x)
    iq_d, iw_d, ik_d = dev(iq), dev(iw), dev(ik)
    pool = torch.full((B * Qn, 2048), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((B * Qn, 512), -7, dtype=torch.int32, device="cuda")
    # the job writes every other row of a larger cache (strided rows)
    codes = torch.full((2 * rows, dim // 2), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((2 * rows, dim // 16), 0x5A, dtype=torch.uint8, device="cuda")
    args = csa2.index_args(iq_d, iw_d, ik_d, Qn)
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    if split:
        csa2.index_scan(args, ws)
        csa2.index_select_append(args, pool, topk, ws, dev(x), codes[::2], scales[::2])
    else:
        csa2.index_full_append(args, pool, topk, ws, dev(x), codes[::2], scales[::2])
    np.testing.assert_array_equal(host(pool), rpool)
    np.testing.assert_array_equal(host(topk), rtopk)
    got_c, got_s = host(codes), host(scales)
    np.testing.assert_array_equal(got_c[::2], rc)
    np.testing.assert_array_equal(got_s[::2], rs)
    assert (got_c[1::2] == 0xA5).all() and (got_s[1::2] == 0x5A).all()
