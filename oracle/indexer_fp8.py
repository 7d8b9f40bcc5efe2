"""Real-valued (FP8) indexer of CSA2 (oracle, FP64).

Test infrastructure only (see the package docstring).

The pages describe the indexer's role (ai-maestro.online, "Compressed Sparse
Attention 2": a Full layer scores the whole context, keeps a pool of 2,048
eight-token blocks and a fresh Top-512; a Reindex layer rescores that pool)
but not the precision of its keys and queries.  The integer indexer
(``indexer``) is the measured configuration; this module is its real-valued
counterpart.  Readings taken:

* R29 indexer keys and queries are OCP E4M3FN codes (the 8-bit format of the
      cache's scales) with fp32 scales: one per position for the keys (its
      D_I channels share it), one per (query, head) for the queries;
* R30 the score is R9 applied to the dequantised values:
          s(q, t) = sum_h w[q, h] * max(0, sq[q, h] * sk[t] * sum_c E4M3(q_hc) * E4M3(k_tc));
* R31 blocks, pool and Top-512 follow R10-R13 and R23 on these scores.  With
      real-valued scores an implementation that evaluates them in fp32 may
      rank two scores closer than its rounding error differently; ``abs_scores``
      gives the magnitude sum that bounds that error.

Arithmetic: every product of two E4M3 values is a multiple of 2^-18 below
2^18, so a dot product over D_I <= 128 channels is an integer multiple of
2^-18 below 2^25: exact in FP64.  The scale products and the head sum round
in FP64 (relative error ~1e-16).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3
from .indexer import BLOCK, POOL_BLOCKS, TOPK, _pad, block_scores, top_ids


def _values(codes) -> np.ndarray:
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def token_scores(iq_q, sq_q, iw_q, ik_rows, sk_rows) -> np.ndarray:
    """s(t) for each row t of ``ik_rows`` (R30).

    iq_q [H_I, D_I] codes, sq_q [H_I], iw_q [H_I], ik_rows [n, D_I] codes, sk_rows [n]."""
    dots = _values(ik_rows) @ _values(iq_q).T                      # [n, H_I], exact
    qk = dots * np.asarray(sk_rows, dtype=np.float64)[:, None] * np.asarray(sq_q, dtype=np.float64)[None, :]
    return (np.maximum(qk, 0.0) * np.asarray(iw_q, dtype=np.float64)[None, :]).sum(axis=1)


def abs_scores(iq_q, sq_q, iw_q, ik_rows, sk_rows) -> np.ndarray:
    """sum_h |w_h| * sq_h * sk_t * sum_c |E4M3(q_hc) * E4M3(k_tc)| per row t:
    the magnitude that bounds the rounding error of any fp32 evaluation of s(t)."""
    dots = np.abs(_values(ik_rows)) @ np.abs(_values(iq_q)).T
    qk = dots * np.abs(np.asarray(sk_rows, dtype=np.float64))[:, None] * np.abs(np.asarray(sq_q, dtype=np.float64))[None, :]
    return (qk * np.abs(np.asarray(iw_q, dtype=np.float64))[None, :]).sum(axis=1)


def full_query(iq_q, sq_q, iw_q, ik_b, sk_b, n_vis: int):
    """Pool (block ids), Top-512 positions and the scores of one Full-layer query."""
    s = token_scores(iq_q, sq_q, iw_q, ik_b[:n_vis], sk_b[:n_vis])
    bs = block_scores(s, n_vis)
    nb = len(bs)
    pool = top_ids(bs, np.arange(nb), min(POOL_BLOCKS, nb))
    cand = (pool[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    cand = cand[cand < n_vis]
    topk = top_ids(s[cand], cand, min(TOPK, len(cand)))
    return pool, topk, s


def index_full(iq, sq, iw, ik, sk, q_per_seq: int, n_visible=None):
    """Full layer: pool [nq, 2048] and Top-512 [nq, 512] (R29-R31, R10-R13).

    iq [nq, H_I, D_I] codes, sq [nq, H_I], iw [nq, H_I], ik [B, T, D_I] codes,
    sk [B, T]; query q belongs to sequence q // q_per_seq."""
    nq = iq.shape[0]
    T = ik.shape[1]
    pools = np.full((nq, POOL_BLOCKS), -1, dtype=np.int32)
    topks = np.full((nq, TOPK), -1, dtype=np.int32)
    for q in range(nq):
        nv = T if n_visible is None else int(n_visible[q])
        b = q // q_per_seq
        pool, topk, _ = full_query(iq[q], sq[q], iw[q], ik[b], sk[b], nv)
        pools[q] = _pad(pool, POOL_BLOCKS)
        topks[q] = _pad(topk, TOPK)
    return pools, topks


def pool_positions(pool_q, n_vis: int) -> np.ndarray:
    """Ascending positions < n_vis of the blocks of one pool row."""
    blocks = np.sort(pool_q[pool_q >= 0].astype(np.int64))
    cand = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    return cand[cand < n_vis]


def reindex_query(iq_q, sq_q, iw_q, ik_b, sk_b, pool_q, n_vis: int):
    """Top-512 of a Reindex layer over the pool's positions, and their scores."""
    cand = pool_positions(pool_q, n_vis)
    s = token_scores(iq_q, sq_q, iw_q, ik_b[cand], sk_b[cand])
    return top_ids(s, cand, min(TOPK, len(cand))), cand, s


def index_reindex(iq, sq, iw, ik, sk, q_per_seq: int, pool, n_visible=None):
    """Reindex layer: Top-512 [nq, 512] from a Full layer's pool [nq, 2048]."""
    nq = iq.shape[0]
    T = ik.shape[1]
    topks = np.full((nq, TOPK), -1, dtype=np.int32)
    for q in range(nq):
        nv = T if n_visible is None else int(n_visible[q])
        b = q // q_per_seq
        topks[q] = _pad(reindex_query(iq[q], sq[q], iw[q], ik[b], sk[b], pool[q], nv)[0], TOPK)
    return topks


def global_topk(iq_q, sq_q, iw_q, ik_b, sk_b, n_vis: int) -> np.ndarray:
    """Top-512 over all visible positions, without the pool (invariant I1)."""
    s = token_scores(iq_q, sq_q, iw_q, ik_b[:n_vis], sk_b[:n_vis])
    return top_ids(s, np.arange(n_vis), min(TOPK, n_vis))
