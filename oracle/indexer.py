"""Hierarchical sparse indexer of CSA2 (oracle, FP64 / exact integers).

Test infrastructure only (see the package docstring).

What the pages fix (ai-maestro.online, "Compressed Sparse Attention 2"):
three per-layer modes.  A Full layer computes indexer keys of its own and
picks a new Top-512; a Reindex layer keeps the preceding Full layer's caches
and candidate set but scores them with a query of its own; a Reuse layer does
no indexing and takes the most recent Top-512.  The Full layer's
hierarchical indexer keeps the 2,048 best 8-token blocks (16,384 positions)
as the candidate set, so a Reindex layer's cost does not grow with the
context.  (The same scheme: wpnews.pro "What is Compressed Sparse Attention 2
CSA2?"; kongchang.com "Three Core Innovations", whose "16,000 blocks" is read
as a garble of 16,384 positions.)

Readings taken for what the pages leave open:

* R9   score s(q, t) = sum_h w[q, h] * max(0, q_h . k_t): one indexer key per
       position shared by all indexer heads, one weight per query and head;
* R10  a block's score is the maximum of its tokens' scores;
* R11  blocks are aligned at position 0; a partial last block uses only its
       visible positions;
* R12  fewer than 2,048 blocks: the pool keeps all of them (padded with -1);
* R13  ranking is by (score descending, position / block id ascending), i.e.
       ties go to the lower index; outputs are ascending, padded with -1;
* R23  the Full layer's Top-512 is taken from its pool (equal to the global
       Top-512, invariant I1, checked by tests).

Scores are exact: the inputs are integers, every product and sum is an
integer far below 2^53, so the FP64 matrix product and sums are exact.
"""
from __future__ import annotations

import numpy as np

TOPK = 512            # Top-512 indices per query token
BLOCK = 8             # tokens per indexer block
POOL_BLOCKS = 2048    # blocks kept by the Full layer (16,384 positions)


def token_scores(iq_q: np.ndarray, iw_q: np.ndarray, ik_rows: np.ndarray) -> np.ndarray:
    """s(t) = sum_h w_h * relu(q_h . k_t) for each row t of ``ik_rows`` (R9)."""
    dots = np.asarray(ik_rows, dtype=np.float64) @ np.asarray(iq_q, dtype=np.float64).T   # [T, H_I]
    return (np.maximum(dots, 0.0) * np.asarray(iw_q, dtype=np.float64)[None, :]).sum(axis=1)


def top_ids(scores: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The k ids ranked first by (score desc, id asc), returned ascending (R13)."""
    order = np.lexsort((ids, -scores))          # primary: -score, secondary: id
    return np.sort(ids[order[:k]])


def _pad(ids: np.ndarray, width: int) -> np.ndarray:
    out = np.full(width, -1, dtype=np.int32)
    out[: len(ids)] = ids
    return out


def block_scores(s: np.ndarray, n_vis: int) -> np.ndarray:
    """Max token score of each 8-token block over visible positions (R10, R11)."""
    nb = (n_vis + BLOCK - 1) // BLOCK
    padded = np.full(nb * BLOCK, -np.inf)
    padded[:n_vis] = s[:n_vis]
    return padded.reshape(nb, BLOCK).max(axis=1)


def full_query(iq_q, iw_q, ik_b, n_vis: int):
    """Pool (block ids) and Top-512 positions of one query of a Full layer."""
    s = token_scores(iq_q, iw_q, ik_b[:n_vis])
    bs = block_scores(s, n_vis)
    nb = len(bs)
    pool = top_ids(bs, np.arange(nb), min(POOL_BLOCKS, nb))
    cand = (pool[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    cand = cand[cand < n_vis]                   # ascending positions
    topk = top_ids(s[cand], cand, min(TOPK, len(cand)))
    return pool, topk, s


def index_full(iq, iw, ik, q_per_seq: int, n_visible=None):
    """Full layer: per query, pool [nq, 2048] (block ids) and Top-512 [nq, 512].

    iq [nq, H_I, D_I] int, iw [nq, H_I], ik [B, T, D_I] int, query q belongs to
    sequence q // q_per_seq; n_visible [nq] (default T) limits each query to
    positions [0, n_visible)."""
    nq = iq.shape[0]
    T = ik.shape[1]
    pools = np.full((nq, POOL_BLOCKS), -1, dtype=np.int32)
    topks = np.full((nq, TOPK), -1, dtype=np.int32)
    for q in range(nq):
        nv = T if n_visible is None else int(n_visible[q])
        pool, topk, _ = full_query(iq[q], iw[q], ik[q // q_per_seq], nv)
        pools[q] = _pad(pool, POOL_BLOCKS)
        topks[q] = _pad(topk, TOPK)
    return pools, topks


def reindex_query(iq_q, iw_q, ik_b, pool_q, n_vis: int):
    """Top-512 of a Reindex layer: rescore only the positions of the pool."""
    blocks = pool_q[pool_q >= 0].astype(np.int64)
    cand = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    cand = cand[cand < n_vis]
    s = token_scores(iq_q, iw_q, ik_b[cand])
    return top_ids(s, cand, min(TOPK, len(cand)))


def index_reindex(iq, iw, ik, q_per_seq: int, pool, n_visible=None):
    """Reindex layer: Top-512 [nq, 512] from the Full layer's pool [nq, 2048]."""
    nq = iq.shape[0]
    T = ik.shape[1]
    topks = np.full((nq, TOPK), -1, dtype=np.int32)
    for q in range(nq):
        nv = T if n_visible is None else int(n_visible[q])
        topks[q] = _pad(reindex_query(iq[q], iw[q], ik[q // q_per_seq], pool[q], nv), TOPK)
    return topks


def global_topk(iq_q, iw_q, ik_b, n_vis: int) -> np.ndarray:
    """Top-512 over all visible positions, without the pool (for invariant I1)."""
    s = token_scores(iq_q, iw_q, ik_b[:n_vis])
    return top_ids(s, np.arange(n_vis), min(TOPK, n_vis))
