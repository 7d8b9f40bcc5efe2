"""Pins of the oracle's hierarchical indexer (CPU only).

Against pure-Python brute force (integer scores, full sorts with tuple keys),
the pool invariant I1 (pool-based Top-512 == global Top-512), the Reindex
invariants I2/I3 and the special cases I4."""
import numpy as np
import pytest

from oracle import indexer


def brute_scores(iq_q, iw_q, ik_b, n):
    out = []
    for t in range(n):
        s = 0
        for h in range(len(iq_q)):
            d = sum(int(a) * int(b) for a, b in zip(iq_q[h], ik_b[t]))
            s += int(iw_q[h]) * max(0, d)
        out.append(s)
    return out


def brute_full(iq_q, iw_q, ik_b, n):
    s = brute_scores(iq_q, iw_q, ik_b, n)
    nb = (n + 7) // 8
    bmax = [max(s[8 * b: min(8 * b + 8, n)]) for b in range(nb)]
    blocks = sorted(range(nb), key=lambda b: (-bmax[b], b))[:2048]
    cand = [8 * b + r for b in sorted(blocks) for r in range(8) if 8 * b + r < n]
    top = sorted(cand, key=lambda t: (-s[t], t))[:512]
    return sorted(blocks), sorted(top)


def _inputs(rng, T, HI, DI, r, wmax, nq=1, B=1):
    iq = rng.integers(-r, r + 1, size=(nq, HI, DI), dtype=np.int8)
    iw = rng.integers(1, wmax + 1, size=(nq, HI)).astype(np.float32)
    ik = rng.integers(-r, r + 1, size=(B, T, DI), dtype=np.int8)
    return iq, iw, ik


@pytest.mark.parametrize("T", [1, 7, 8, 9, 63, 511, 512, 513, 1000])
def test_brute_force_small(T):
    rng = np.random.default_rng(T)
    iq, iw, ik = _inputs(rng, T, 2, 8, 1, 2)          # narrow ranges: many ties
    pool, topk = indexer.index_full(iq, iw, ik, 1)
    bpool, btop = brute_full(iq[0], iw[0], ik[0], T)
    assert list(pool[0][pool[0] >= 0]) == bpool
    assert list(topk[0][topk[0] >= 0]) == btop
    assert np.all(pool[0][len(bpool):] == -1) and np.all(topk[0][len(btop):] == -1)


def test_brute_force_pool_selection_with_ties():
    # T > 16,384 so that the pool actually drops blocks; tiny value range -> heavy ties
    T = 20000
    rng = np.random.default_rng(5)
    iq, iw, ik = _inputs(rng, T, 2, 4, 1, 1)
    pool, topk = indexer.index_full(iq, iw, ik, 1)
    bpool, btop = brute_full(iq[0], iw[0], ik[0], T)
    assert list(pool[0]) == bpool
    assert list(topk[0]) == btop


@pytest.mark.parametrize("seed", range(4))
def test_invariant_pool_topk_equals_global(seed):
    T = 40000
    rng = np.random.default_rng(100 + seed)
    iq, iw, ik = _inputs(rng, T, 8, 16, 2 + seed, 3)
    pool, topk = indexer.index_full(iq, iw, ik, 1)
    glob = indexer.global_topk(iq[0], iw[0], ik[0], T)
    np.testing.assert_array_equal(topk[0], glob)


def test_reindex_invariants():
    T = 30000
    rng = np.random.default_rng(9)
    iq, iw, ik = _inputs(rng, T, 4, 16, 3, 4, nq=3, B=3)
    pool, topk = indexer.index_full(iq, iw, ik, 1)
    # I3: reindex with the Full layer's own q and w reproduces its Top-512
    np.testing.assert_array_equal(indexer.index_reindex(iq, iw, ik, 1, pool), topk)
    # I2: a different q selects only pool positions
    iq2, iw2, _ = _inputs(rng, T, 4, 16, 3, 4, nq=3, B=3)
    t2 = indexer.index_reindex(iq2, iw2, ik, 1, pool)
    for q in range(3):
        blocks = set(pool[q][pool[q] >= 0].tolist())
        assert all((t // 8) in blocks for t in t2[q] if t >= 0)
        # and it equals brute force over the pool's positions
        cand = [8 * b + r for b in sorted(blocks) for r in range(8)]
        s = brute_scores(iq2[q], iw2[q], ik[q][cand], len(cand))
        best = sorted(range(len(cand)), key=lambda i: (-s[i], cand[i]))[:512]
        assert list(t2[q]) == sorted(cand[i] for i in best)


def test_special_cases():
    T = 20000
    rng = np.random.default_rng(1)
    _, iw, ik = _inputs(rng, T, 2, 8, 4, 4)
    zero_q = np.zeros((1, 2, 8), dtype=np.int8)
    pool, topk = indexer.index_full(zero_q, iw, ik, 1)       # all scores equal
    np.testing.assert_array_equal(pool[0], np.arange(2048))
    np.testing.assert_array_equal(topk[0], np.arange(512))
    # strictly increasing scores: k_t = t (one channel), q = 1 -> last 512 positions
    Tn = 5000
    ik2 = np.zeros((1, Tn, 8), dtype=np.int64)
    ik2[0, :, 0] = np.arange(Tn)
    q1 = np.zeros((1, 1, 8), dtype=np.int64)
    q1[0, 0, 0] = 1
    pool, topk = indexer.index_full(q1, np.ones((1, 1)), ik2, 1)
    np.testing.assert_array_equal(topk[0], np.arange(Tn - 512, Tn))
    # T < 512: every position, then -1 padding
    pool, topk = indexer.index_full(zero_q, iw, ik[:, :300], 1)
    np.testing.assert_array_equal(topk[0][:300], np.arange(300))
    assert np.all(topk[0][300:] == -1)
    assert list(pool[0][:38]) == list(range(38)) and np.all(pool[0][38:] == -1)


def test_n_visible_limits_positions():
    T = 3000
    rng = np.random.default_rng(4)
    iq, iw, ik = _inputs(rng, T, 2, 8, 2, 3, nq=2, B=1)
    nv = np.array([1234, 0])
    pool, topk = indexer.index_full(iq, iw, ik, 2, n_visible=nv)
    bpool, btop = brute_full(iq[0], iw[0], ik[0], 1234)
    assert list(topk[0][topk[0] >= 0]) == btop
    assert np.all(topk[1] == -1) and np.all(pool[1] == -1)


@pytest.mark.parametrize("seed,T,r", [(0, 40000, 2), (1, 40000, 1), (2, 6000, 0), (3, 4500, 3), (4, 3000, 1)])
def test_top512_lies_in_top512_blocks(seed, T, r):
    """The pruning the GPU selection uses, checked on the oracle's scores: the
    Top-512 positions lie in the top min(512, #blocks) blocks (by block max,
    ties to the lower block), and when there are at least 512 blocks every
    selected score is >= the 512th block score, so candidates below it can be
    dropped.  (T = 3000 and 4500 have fewer than 512 blocks but more than 512
    positions; r = 0 makes every score equal.)"""
    rng = np.random.default_rng(300 + seed)
    iq, iw, ik = _inputs(rng, T, 8, 16, r, 3)
    _, topk, s = indexer.full_query(iq[0], iw[0], ik[0], T)
    bs = indexer.block_scores(s, T)
    nb = len(bs)
    k = min(512, nb)
    top_blocks = indexer.top_ids(bs, np.arange(nb), k)
    assert set((topk // 8).tolist()) <= set(top_blocks.tolist())
    if nb >= 512:
        kth = np.sort(bs)[::-1][511]                 # the 512th block score
        assert s[topk].min() >= kth
    # the pruned candidate set gives the same Top-512 as the full pool
    cand = (top_blocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    cand = cand[cand < T]
    if nb >= 512:
        cand = cand[s[cand] >= np.sort(bs)[::-1][511]]
    np.testing.assert_array_equal(indexer.top_ids(s[cand], cand, min(512, len(cand))), topk)
