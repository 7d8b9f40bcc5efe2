"""Helpers for the GPU parity tests: device upload, oracle-side reconstruction
of the synthetic workloads and the attention error metric.

Expected values always come from the oracle run on the seeded inputs (never
from the HIP path)."""
from __future__ import annotations

import numpy as np
import torch

from fp4_kv_cache_e4m3_amd import synth
from oracle import attention as oattn
from oracle import indexer as oidx
from oracle import quant as oquant
from oracle import swa8 as oswa8

ATTN_TOL = 2e-3     # max over (query, head) of max_c |O - O_ref| / max_c |O_ref|


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rownorm_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Row-normalised infinity-norm error per (query, head), maximised."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def oracle_index_full(w: synth.Workload, iq, iw, ik, n_visible=None):
    return oidx.index_full(iq, iw, ik, w.q_per_seq, n_visible)


def oracle_kv_rows(w: synth.Workload, b: int, positions: np.ndarray, with_new_rows: bool = True):
    """Oracle FP4 codes/scales of sequence b's rows ``positions`` as the cache
    holds them after one step (rows T - new_per_seq .. T - 1 = the step's new
    entries)."""
    positions = np.asarray(positions, dtype=np.int64)
    src = np.empty((len(positions), w.dim), dtype=np.float32)
    order = np.argsort(positions)
    sp = positions[order]
    # regenerate only the seeded chunks that hold the requested rows
    chunks = np.unique(sp // synth.KV_CHUNK_ROWS)
    buf = {}
    for c in chunks:
        r0 = int(c) * synth.KV_CHUNK_ROWS
        n = min(synth.KV_CHUNK_ROWS, w.kv_len - r0)
        buf[int(c)] = synth.kv_source_rows(w, b, r0, n)
    for i, p in zip(order, sp):
        src[i] = buf[int(p // synth.KV_CHUNK_ROWS)][int(p % synth.KV_CHUNK_ROWS)]
    if with_new_rows:
        n = w.new_per_seq
        nr = synth.new_rows(w)[b * n:(b + 1) * n]
        sel = positions >= w.kv_len - n
        src[sel] = nr[positions[sel] - (w.kv_len - n)]
    return oquant.quantize_rows(src)


def oracle_selected_rows(w: synth.Workload, topk, queries, with_new_rows=True) -> dict:
    """Oracle FP4 codes/scales of the rows each query's Top-K names:
    {query: (codes, scales)} in Top-K order.  The rows of one sequence are
    quantised once over the union of its queries' positions, so the seeded
    chunks are regenerated once per sequence (layers sharing a Top-K reuse
    the result)."""
    out = {}
    by_seq = {}
    for qi in queries:
        by_seq.setdefault(qi // w.q_per_seq, []).append(qi)
    for b, qis in by_seq.items():
        allpos = np.unique(np.concatenate([topk[qi][topk[qi] >= 0].astype(np.int64) for qi in qis]))
        codes, scales = oracle_kv_rows(w, b, allpos, with_new_rows)
        for qi in qis:
            idx = np.searchsorted(allpos, topk[qi][topk[qi] >= 0].astype(np.int64))
            out[qi] = (codes[idx], scales[idx])
    return out


def oracle_attention(w: synth.Workload, q_bits, swa_bits, topk, with_new_rows=True, queries=None,
                     swa_len=None, rows=None):
    """Oracle output of one layer for the given Top-K (oracle's own), [nq, H, d].
    rows: optional precomputed oracle_selected_rows for the same Top-K."""
    nq = w.nq
    qsel = range(nq) if queries is None else queries
    out = np.zeros((nq, w.heads, w.dim))
    qv = bf16_values(q_bits)
    sv = bf16_values(swa_bits)
    if w.swa8:                           # the window as its 8-bit rows hold it
        rc, rs = oswa8.quantize_swa_rows(sv.reshape(-1, w.dim))
        sv = oswa8.swa_values(rc, rs).reshape(sv.shape)
    if rows is None:
        rows = oracle_selected_rows(w, topk, list(qsel), with_new_rows)
    for qi in qsel:
        b = qi // w.q_per_seq
        pos = topk[qi][topk[qi] >= 0].astype(np.int64)
        codes, scales = rows[qi]
        # local cache holding just these rows: row i <-> position pos[i]
        local_topk = np.arange(len(pos), dtype=np.int64)
        keys = oattn.query_entries(qi % w.q_per_seq, w.q_per_seq, len(pos), local_topk, codes, scales,
                                   sv[b:b + 1], w.window,
                                   None if swa_len is None else np.asarray(swa_len)[b:b + 1])
        out[qi] = oattn.attend(qv[qi], keys, 1.0 / np.sqrt(w.dim))
    return out
