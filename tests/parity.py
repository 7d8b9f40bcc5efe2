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


def window_bits(w: synth.Workload, layer: int) -> np.ndarray:
    """bf16 window rows of a layer as a step leaves them: with 8-bit windows
    the step writes its query tokens' new rows into the newest slots."""
    bits = synth.swa_bf16(w, layer)
    if w.swa8:
        nb = synth.new_swa_rows(w, layer).reshape(w.batch, w.q_per_seq, w.dim)
        bits[:, w.swa_rows - w.q_per_seq:] = nb
    return bits


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


# ---------------------------------------------------------------- FP8 indexer
U32 = 2.0 ** -24


def fp8_score_bound(abs_s: np.ndarray, dim: int, heads: int) -> np.ndarray:
    """Largest |fp32 evaluation - exact score| of an FP8 indexer score whose
    magnitude sum (oracle.indexer_fp8.abs_scores) is abs_s: D_I products
    summed (at most D_I - 1 roundings), the weight times query-scale product,
    the weighted head sum (H_I - 1 roundings), the key-scale product and one
    rounding of the weighted term each stay within (D_I + H_I + 4) units of
    2^-24 of the magnitude sum, whatever the summation order."""
    return (dim + heads + 4) * U32 * np.asarray(abs_s, dtype=np.float64)


def keys_to_scores(keys: np.ndarray) -> np.ndarray:
    """fp32 scores of the library's order-preserving uint32 ranking keys."""
    k = np.asarray(keys, dtype=np.uint32)
    bits = np.where(k & np.uint32(0x80000000), k & np.uint32(0x7FFFFFFF), ~k).astype(np.uint32)
    return bits.view(np.float32).astype(np.float64)


def _selection_errors(sel_row, cand, s_of, e_of, k, what):
    errs = []
    sel = sel_row[sel_row >= 0].astype(np.int64)
    if not np.all(sel_row[len(sel):] == -1):
        errs.append(f"{what}: padding is not trailing -1")
    if len(sel) != min(k, len(cand)):
        errs.append(f"{what}: {len(sel)} entries, expected {min(k, len(cand))}")
    if len(sel) > 1 and np.any(np.diff(sel) <= 0):
        errs.append(f"{what}: not strictly ascending")
    if not np.all(np.isin(sel, cand)):
        errs.append(f"{what}: entries outside the candidates")
        return errs
    rest = np.setdiff1d(cand, sel)
    if len(sel) and len(rest):
        lo = (s_of(sel) + e_of(sel)).min()
        hi = (s_of(rest) - e_of(rest)).max()
        if lo < hi:
            errs.append(f"{what}: a dropped candidate outranks a selected one beyond the rounding bound "
                        f"({lo!r} < {hi!r})")
    return errs


def fp8_full_errors(pool_row, topk_row, s: np.ndarray, eps: np.ndarray, n_vis: int):
    """Problems with a Full layer's pool / Top-512 row given the oracle's exact
    scores s and bounds eps of positions [0, n_vis): each must be a valid
    selection for some scores within eps of the exact ones (blocks by their
    maxima, positions among the pool's), in the library's output format."""
    nb = (n_vis + 7) // 8
    sp = np.full(nb * 8, -np.inf)
    sp[:n_vis] = s[:n_vis]
    ep = np.zeros(nb * 8)
    ep[:n_vis] = eps[:n_vis]
    bmax = sp.reshape(nb, 8).max(axis=1)
    bep = ep.reshape(nb, 8).max(axis=1)
    errs = _selection_errors(np.asarray(pool_row), np.arange(nb), lambda i: bmax[i], lambda i: bep[i],
                             2048, "pool")
    if errs:
        return errs
    blocks = pool_row[pool_row >= 0].astype(np.int64)
    cand = (blocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    cand = cand[cand < n_vis]
    return _selection_errors(np.asarray(topk_row), cand, lambda i: s[i], lambda i: eps[i], 512, "top-512")


def fp8_topk_errors(topk_row, cand: np.ndarray, s_cand: np.ndarray, e_cand: np.ndarray):
    """Problems with a Reindex Top-512 row over candidate positions cand
    (ascending) with exact scores s_cand and bounds e_cand."""
    pos = {int(p): i for i, p in enumerate(cand)}
    idx = lambda ps: np.array([pos[int(p)] for p in ps], dtype=np.int64)
    return _selection_errors(np.asarray(topk_row), cand, lambda ps: s_cand[idx(ps)],
                             lambda ps: e_cand[idx(ps)], 512, "top-512")
