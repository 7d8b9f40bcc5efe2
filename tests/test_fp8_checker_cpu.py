"""The FP8-indexer selection checker of the GPU parity tests (CPU only): it
accepts the oracle's own selections and rejects planted mistakes (planted in
oracle results, on the CPU)."""
import numpy as np
import pytest

from oracle import indexer_fp8
from tests.parity import fp8_full_errors, fp8_score_bound, fp8_topk_errors, keys_to_scores


def _case(seed, T=30000, HI=4, DI=64):
    rng = np.random.default_rng(seed)
    cq = rng.integers(0, 0x7F, size=(HI, DI)).astype(np.uint8) | (rng.integers(0, 2, size=(HI, DI)) << 7).astype(np.uint8)
    ck = rng.integers(0, 0x7F, size=(T, DI)).astype(np.uint8) | (rng.integers(0, 2, size=(T, DI)) << 7).astype(np.uint8)
    sq = (rng.random(HI) + 0.5).astype(np.float32)
    sk = (rng.random(T) + 0.5).astype(np.float32)
    iw = (rng.random(HI) * 1.25 - 0.25).astype(np.float32)
    s = indexer_fp8.token_scores(cq, sq, iw, ck, sk)
    eps = fp8_score_bound(indexer_fp8.abs_scores(cq, sq, iw, ck, sk), DI, HI)
    pool, topk, _ = indexer_fp8.full_query(cq, sq, iw, ck, sk, T)
    prow = np.full(2048, -1, np.int32)
    prow[:len(pool)] = pool
    trow = np.full(512, -1, np.int32)
    trow[:len(topk)] = topk
    return s, eps, prow, trow, T


@pytest.mark.parametrize("seed", [0, 1])
def test_accepts_oracle_selection(seed):
    s, eps, prow, trow, T = _case(seed)
    assert fp8_full_errors(prow, trow, s, eps, T) == []
    # an ulp-level perturbation inside the bound is still accepted
    assert fp8_full_errors(prow, trow, s * (1 + 1e-9), eps, T) == []


def test_rejects_planted_mistakes():
    s, eps, prow, trow, T = _case(2)
    # a selected position swapped for the worst candidate of the pool
    blocks = prow[prow >= 0].astype(np.int64)
    cand = (blocks[:, None] * 8 + np.arange(8)).reshape(-1)
    rest = np.setdiff1d(cand, trow)
    bad = trow.copy()
    bad[0] = rest[np.argmin(s[rest])]
    bad[:512] = np.sort(bad[:512])
    assert any("outranks" in e for e in fp8_full_errors(prow, bad, s, eps, T))
    # a pool block swapped for the lowest-scoring block outside it
    nb = (T + 7) // 8
    bmax = s[:nb * 8].reshape(nb, 8).max(axis=1)
    out = np.setdiff1d(np.arange(nb), blocks)
    bp = prow.copy()
    bp[0] = out[np.argmin(bmax[out])]
    bp[:2048] = np.sort(bp[:2048])
    assert any("pool" in e for e in fp8_full_errors(bp, trow, s, eps, T))
    # format: unsorted, short, bad padding
    uns = trow.copy()
    uns[[0, 1]] = uns[[1, 0]]
    assert any("ascending" in e for e in fp8_full_errors(prow, uns, s, eps, T))
    short = trow.copy()
    short[-1] = -1
    assert any("entries" in e for e in fp8_full_errors(prow, short, s, eps, T))
    # the reindex form of the check
    sc = s[cand]
    ec = eps[cand]
    good = np.full(512, -1, np.int32)
    order = np.lexsort((cand, -sc))[:512]
    good[:] = np.sort(cand[order])
    assert fp8_topk_errors(good, cand, sc, ec) == []
    wrong = good.copy()
    wrong[0] = np.setdiff1d(cand, good)[np.argmin(s[np.setdiff1d(cand, good)])]
    wrong = np.sort(wrong)
    assert any("outranks" in e for e in fp8_topk_errors(wrong, cand, sc, ec))


def test_keys_to_scores_known_values():
    keys = np.array([0x80000000, 0x80000000 | 0x3F800000, 0x407FFFFF, 0x80000000 | 0x7F7FFFFF], dtype=np.uint32)
    assert list(keys_to_scores(keys)) == [0.0, 1.0, -1.0, float(np.finfo(np.float32).max)]
