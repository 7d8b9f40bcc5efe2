"""Sparse Top-K + sliding-window attention of one CSA2 layer (oracle, FP64).

Test infrastructure only (see the package docstring).

What the pages fix: each layer attends with a query and a local-window
cache of its own (ai-maestro.online, "Compressed Sparse Attention 2"); the
local window covers the latest 128 tokens (same page, "Causal
Encoder-Decoder architecture"); the sparse entries are the Top-512 list the
layer's mode supplies (Full and Reindex layers make a new one, Reuse layers
take the most recent); main-cache entries are E2M1 values with an E4M3
multiplier per 16 channels.

Readings taken for what the pages leave open:

* R14  one d-vector per entry is both key and value (main cache and SWA);
* R15  query j of a sequence sees SWA buffer rows j .. j+W-1, i.e. the W
       tokens ending at itself; the buffer holds W-1+Qn rows per sequence;
* R16  every query sees all entries its Top-K list names;
* R18  the Top-K entries and the SWA rows are concatenated without dedup and
       share one softmax;
* R19  logits are scaled by 1/sqrt(d) unless another scale is given;
* R24  output is fp32-representable FP64 here (the kernel writes fp32).

An empty Top-K slot (-1) contributes nothing; an SWA row before the
sequence's first valid row (``swa_len``) contributes nothing; a query with no
entry at all gets a zero output.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import dequant_rows


def attend(qh: np.ndarray, keys: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * Q K^T) K for one query: qh [H, d], keys [n, d] (V = K)."""
    if keys.shape[0] == 0:
        return np.zeros_like(qh)
    logits = sm_scale * (qh @ keys.T)                 # [H, n]
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    return (p @ keys) / p.sum(axis=1, keepdims=True)


def query_entries(q, q_per_seq, kv_len, topk_q, codes, scales, swa, window, swa_len=None):
    """FP64 rows the query attends to: dequantised Top-K rows, then its SWA rows."""
    b, j = divmod(q, q_per_seq)
    dim = swa.shape[-1]
    pos = np.asarray(topk_q, dtype=np.int64)
    pos = pos[(pos >= 0) & (pos < kv_len)]
    rows = b * kv_len + pos
    sparse = dequant_rows(codes[rows], scales[rows], dim)
    nrows = swa.shape[1]
    first = 0 if swa_len is None else nrows - int(swa_len[b])
    r = np.arange(j, j + window)
    r = r[(r >= first) & (r < nrows)]
    return np.concatenate([sparse, np.asarray(swa[b, r], dtype=np.float64)], axis=0)


def sparse_attn(q, codes, scales, topk, swa, q_per_seq: int, kv_len: int,
                window: int = 128, sm_scale: float | None = None, swa_len=None,
                queries=None) -> np.ndarray:
    """Output [nq, H, d] (FP64) of one CSA2 attention layer.

    q [nq, H, d] (values of the bf16 queries), codes [B*T, d/2] / scales
    [B*T, d/16] (the FP4 main KV, row b*T + t), topk [nq, k] positions
    (-1 = empty), swa [B, W-1+Qn, d] (values of the bf16 window rows).
    ``queries`` restricts the work to a subset (other rows stay zero)."""
    q = np.asarray(q, dtype=np.float64)
    nq, H, dim = q.shape
    scale = 1.0 / math.sqrt(dim) if not sm_scale else float(sm_scale)
    out = np.zeros_like(q)
    for qi in (range(nq) if queries is None else queries):
        keys = query_entries(qi, q_per_seq, kv_len, topk[qi], codes, scales, swa, window, swa_len)
        out[qi] = attend(q[qi], keys, scale)
    return out
