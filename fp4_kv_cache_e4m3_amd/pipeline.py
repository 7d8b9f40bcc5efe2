"""One CSA2 layer group on the device: staging of a synthetic workload and the
ordered library calls of one decode / prefill step.

The call order follows the pages' layer schedule (ai-maestro.online,
"Compressed Sparse Attention 2"): a group starts with a Full layer (own FP4
main KV, fresh indexer scan, pool + Top-512) or a Reindex layer (rescore the
last Full layer's pool with its own indexer Q), followed by Reuse layers that
attend with their own Q and sliding window over the latest Top-K.  Every
step's computation runs in libcsa2.so; this module only allocates buffers and
issues the C-ABI calls.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as B
from . import synth


def _dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device, non_blocking=False)


class DecodeGroup:
    """Device state of a synthetic sequence of CSA2 layers and its step.

    ``w.layers`` names the layers, e.g. ("full", "reuse", "reuse", "reuse"),
    ("reindex", "reuse", ...) or a whole decoder (a Full group followed by
    Reindex groups).  A Full layer quantises the step's new main-KV rows and
    runs the Full indexer (pool + Top-K); a Reindex layer rescores the latest
    pool with its own indexer Q; a Reuse layer attends with the latest Top-K.
    Each indexing layer writes its own Top-K buffer (``topks[i]``).  When the
    sequence starts with a Reindex layer, the pool of the Full layer before it
    is produced once at set-up (from the pool-source indexer Q) and is an
    input of every step."""

    def __init__(self, w: synth.Workload, device: str = "cuda", kv_rows=None, fused_window: bool = True,
                 rows_once: bool = True):
        self.w = w
        self.device = device
        dev = device
        B_, T, d = w.batch, w.kv_len, w.dim
        # ---- FP4 main KV cache: quantised on the device from seeded fp32 rows,
        # contiguous [B * T] rows or (paged) pages named by a block table
        P = w.page_size
        self.block_table_host = synth.block_table(w) if P else None
        self.block_table = _dev(self.block_table_host, dev) if P else None
        n_rows = synth.page_count(w)[1] * P if P else B_ * T
        self.codes = torch.empty((n_rows, d // 2), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((n_rows, d // 16), dtype=torch.uint8, device=dev)
        chunk = 65536
        for b in range(B_):
            for r0 in range(0, T, chunk):
                n = min(chunk, T - r0)
                src = _dev(synth.kv_source_rows(w, b, r0, n), dev)
                if P:
                    seq = torch.full((n,), b, dtype=torch.int32, device=dev)
                    pos = torch.arange(r0, r0 + n, dtype=torch.int32, device=dev)
                    B.quantize_kv_paged(src, seq, pos, self.block_table, P, self.codes, self.scales)
                    torch.cuda.synchronize()
                    del seq, pos
                else:
                    base = b * T + r0
                    B.quantize_kv(src, self.codes[base:base + n], self.scales[base:base + n])
                del src
        # ---- indexer keys [B, T, D_I] (int8, or E4M3 codes with [B, T] scales)
        self.ik = torch.empty((B_, T, w.idx_dim), dtype=torch.uint8 if w.idx_fp8 else torch.int8, device=dev)
        for b in range(B_):
            self.ik[b].copy_(torch.from_numpy(synth.index_k(w, b)))
        self.ik_scale = _dev(synth.index_k_scale_all(w), dev) if w.idx_fp8 else None
        # ---- per-step inputs
        self.new_rows = _dev(synth.new_rows(w), dev)           # [B * new_per_seq, d] fp32
        nl = len(w.layers)
        # indexing layers (Full / Reindex) and, per layer, the Top-K it reads
        self.index_layers = [l for l, m in enumerate(w.layers) if m in ("full", "reindex")]
        assert self.index_layers and self.index_layers[0] == 0, "the first layer must index"
        qs = (lambda l, src=False: _dev(synth.index_q_scale(w, l, src), dev)) if w.idx_fp8 else (lambda l, src=False: None)
        self.iq = _dev(synth.index_q(w, 0), dev)
        self.iw = _dev(synth.index_w(w, 0), dev)
        self._iqw = {0: (self.iq, self.iw, qs(0))}
        for l in self.index_layers[1:]:
            self._iqw[l] = (_dev(synth.index_q(w, l), dev), _dev(synth.index_w(w, l), dev), qs(l))
        self.q = [_dev(synth.attn_q_bf16(w, l).view(np.int16), dev) for l in range(nl)]
        # windows: linear [B, W - 1 + Qn] rows, or a ring whose row r of
        # sequence b sits in slot (start[b] + r) mod rows
        self.swa_start = [None] * nl
        self.swa = []
        for l in range(nl):
            rows = synth.swa_bf16(w, l)
            if w.swa_ring:
                st = synth.swa_ring_start(w, l)
                rows = np.stack([np.roll(rows[b], int(st[b]), axis=0) for b in range(B_)])
                self.swa_start[l] = _dev(st, dev)
            self.swa.append(_dev(np.ascontiguousarray(rows).view(np.int16), dev))
        # 8-bit window rows: the older rows quantised once on the device from
        # the bf16 rows; each step encodes its query tokens' new rows into
        # the newest slots (rows swa_rows - Qn .. swa_rows - 1): inside the
        # attention call (fused_window), or by one strided quantise call per
        # query slot before it
        self.swa_scale = [None] * nl
        self._swa_new = [[] for _ in range(nl)]
        self._swa_rows_new = [None] * nl
        assert not (w.swa8 and w.swa_ring), "8-bit rings are not set up here"
        if w.swa8:
            for l in range(nl):
                codes8 = torch.empty((B_, w.swa_rows, d), dtype=torch.uint8, device=dev)
                sc8 = torch.empty((B_, w.swa_rows), dtype=torch.float32, device=dev)
                B.quantize_swa_fp8(self.swa[l].view(B_ * w.swa_rows, d), codes8.view(B_ * w.swa_rows, d), sc8.view(-1))
                self.swa[l], self.swa_scale[l] = codes8, sc8
                nb = _dev(synth.new_swa_rows(w, l).view(np.int16), dev).view(B_, w.q_per_seq, d)
                if fused_window:
                    self._swa_rows_new[l] = nb.view(B_ * w.q_per_seq, d)
                    continue
                for i in range(w.q_per_seq):          # one strided call per query slot
                    r = w.swa_rows - w.q_per_seq + i
                    self._swa_new[l].append((nb[:, i, :], codes8[:, r, :], sc8[:, r]))
        # ---- outputs and workspaces
        nq = w.nq
        self.pool = torch.full((nq, B.POOL_BLOCKS), -1, dtype=torch.int32, device=dev)
        self.topks = [torch.full((nq, B.TOPK), -1, dtype=torch.int32, device=dev) for _ in self.index_layers]
        self.topk = self.topks[0]
        self.out = [torch.empty((nq, w.heads, d), dtype=torch.float32, device=dev) for _ in range(nl)]
        self.iargs_by_layer = {l: B.index_args(iq, iw, self.ik, w.q_per_seq, q_scale=sq, k_scale=self.ik_scale)
                               for l, (iq, iw, sq) in self._iqw.items()}
        self.iargs = self.iargs_by_layer[0]
        self.iws = torch.empty(max(256, B.index_workspace_size(self.iargs)), dtype=torch.uint8, device=dev)
        # Top-K buffer of each layer: the latest indexing layer's
        self._topk_of = []
        k = -1
        for m in w.layers:
            k += m in ("full", "reindex")
            self._topk_of.append(self.topks[k])
        # Paged cache (rows_once): an indexing layer's attention call also
        # writes its Top-K as cache rows, and the later layers that share
        # that Top-K read the rows (no block-table reads of their own)
        self.aargs = []
        rows_of = {}
        for l, m in enumerate(w.layers):
            tk = self._topk_of[l]
            kw = dict(swa_scale=self.swa_scale[l], swa_start=self.swa_start[l], swa_new=self._swa_rows_new[l])
            if P and rows_once and m in ("full", "reindex"):
                rows_of[id(tk)] = torch.full_like(tk, -1)
                kw.update(block_table=self.block_table, page_size=P, topk_rows_out=rows_of[id(tk)])
            elif P and rows_once and id(tk) in rows_of:
                tk = rows_of[id(tk)]
                kw.update(topk_is_rows=True)
            else:
                kw.update(block_table=self.block_table, page_size=P)
            self.aargs.append(B.attn_args(self.q[l], self.codes, self.scales, tk, self.swa[l], self.out[l],
                                          w.q_per_seq, T, w.window, **kw))
        aws = max(B.attn_workspace_size(a) for a in self.aargs)
        self.aws = torch.empty(max(256, aws), dtype=torch.uint8, device=dev) if aws > 0 else None
        # a step's new entries land in the last new_per_seq slots of each
        # sequence (rows b*T + T - n + i); one strided quantise call per
        # sequence or per slot index, whichever is fewer
        n = w.new_per_seq
        self._new_calls = []
        self._new_paged = None
        # several new rows in each of several sequences of a contiguous
        # cache: the cache is a paged one whose block table maps page i of
        # sequence b to page b * (T / P) + i (P the largest power of two
        # <= 65,536 dividing T), so the rows go out in one job of the
        # selection launch
        P_id = min(T & -T, 65536)
        if P:                                   # one call: rows through the block table
            self._new_paged = (self.new_rows,
                               _dev(np.repeat(np.arange(B_, dtype=np.int32), n), dev),
                               _dev(np.tile(np.arange(T - n, T, dtype=np.int32), B_), dev),
                               self.block_table, P)
        elif n > 1 and B_ > 1 and P_id >= 64:
            pages = T // P_id
            table = (np.arange(B_, dtype=np.int32)[:, None] * pages + np.arange(pages, dtype=np.int32)[None, :])
            self._new_paged = (self.new_rows,
                               _dev(np.repeat(np.arange(B_, dtype=np.int32), n), dev),
                               _dev(np.tile(np.arange(T - n, T, dtype=np.int32), B_), dev),
                               _dev(table, dev), P_id)
        elif n == 1:
            self._new_calls.append((self.new_rows, self.codes[T - 1::T], self.scales[T - 1::T]))
        elif B_ <= n:
            for b in range(B_):
                r = slice(b * T + T - n, b * T + T)
                self._new_calls.append((self.new_rows[b * n:(b + 1) * n], self.codes[r], self.scales[r]))
        else:
            for i in range(n):
                self._new_calls.append((self.new_rows[i::n], self.codes[T - n + i::T], self.scales[T - n + i::T]))
        if w.layers[0] == "reindex":
            iq0 = _dev(synth.index_q(w, 0, pool_source=True), dev)
            iw0 = _dev(synth.index_w(w, 0, pool_source=True), dev)
            sq0 = qs(0, True)
            pa = B.index_args(iq0, iw0, self.ik, w.q_per_seq, q_scale=sq0, k_scale=self.ik_scale)
            scratch = torch.empty_like(self.topk)
            B.index_full(pa, self.pool, scratch, self.iws)
            self._pool_src = (iq0, iw0, sq0)
        torch.cuda.synchronize()

    # the stages of one step (bench.py times them apart)
    def quantize_new(self, stream=None) -> None:
        if self._new_paged is not None:
            x, seq, pos, bt, page = self._new_paged
            B.quantize_kv_paged(x, seq, pos, bt, page, self.codes, self.scales, stream)
        for x, c, s in self._new_calls:
            B.quantize_kv(x, c, s, stream)

    def quantize_window(self, l: int, stream=None) -> None:
        """8-bit windows: the step's new window rows of layer l into their slots."""
        for x, c, s in self._swa_new[l]:
            B.quantize_swa_fp8(x, c, s, stream)

    def cache_rows(self, b: int, positions) -> np.ndarray:
        """Rows of codes / scales holding sequence b's positions."""
        positions = np.asarray(positions, dtype=np.int64)
        if not self.w.page_size:
            return b * self.w.kv_len + positions
        P = self.w.page_size
        return self.block_table_host[b, positions // P].astype(np.int64) * P + positions % P

    def pool_out(self):
        """The pool buffer, or None for an encoder group (no Reindex consumes it)."""
        return None if self.w.encoder else self.pool

    def calls(self, stream=None, split_full: bool = False) -> list:
        """The ordered library calls of one step as (stage, callable) pairs;
        stages: quantize, index_full (or index_scan + index_select with
        split_full), reindex, attention."""
        out = []
        for l, m in enumerate(self.w.layers):
            if m == "full" and self._new_paged is not None:
                # the new rows go through a block table (the cache's own, or
                # the identity table of a contiguous cache), as extra
                # workgroups of the selection launch
                ia, tk = self.iargs_by_layer[l], self._topk_of[l]
                x, seq, pos, bt, page = self._new_paged
                pg = (x, seq, pos, bt, page, self.codes, self.scales)
                if split_full:
                    out.append(("index_scan", lambda ia=ia: B.index_scan(ia, self.iws, stream)))
                    out.append(("index_select", lambda ia=ia, tk=tk, pg=pg: B.index_select_append_paged(
                        ia, self.pool_out(), tk, self.iws, *pg, stream)))
                else:
                    out.append(("index_full", lambda ia=ia, tk=tk, pg=pg: B.index_full_append_paged(
                        ia, self.pool_out(), tk, self.iws, *pg, stream)))
            elif m == "full" and len(self._new_calls) == 1:
                # one strided job: the new rows are quantised by the Full
                # layer's selection launch itself
                ia, tk = self.iargs_by_layer[l], self._topk_of[l]
                x, c, sc = self._new_calls[0]
                if split_full:
                    out.append(("index_scan", lambda ia=ia: B.index_scan(ia, self.iws, stream)))
                    out.append(("index_select", lambda ia=ia, tk=tk: B.index_select_append(
                        ia, self.pool_out(), tk, self.iws, x, c, sc, stream)))
                else:
                    out.append(("index_full", lambda ia=ia, tk=tk: B.index_full_append(
                        ia, self.pool_out(), tk, self.iws, x, c, sc, stream)))
            elif m == "full":
                ia, tk = self.iargs_by_layer[l], self._topk_of[l]
                out.append(("quantize", lambda: self.quantize_new(stream)))
                if split_full:
                    out.append(("index_scan", lambda ia=ia: B.index_scan(ia, self.iws, stream)))
                    out.append(("index_select",
                                lambda ia=ia, tk=tk: B.index_select(ia, self.pool_out(), tk, self.iws, stream)))
                else:
                    out.append(("index_full",
                                lambda ia=ia, tk=tk: B.index_full(ia, self.pool_out(), tk, self.iws, stream)))
            elif m == "reindex":
                ia, tk = self.iargs_by_layer[l], self._topk_of[l]
                out.append(("reindex", lambda ia=ia, tk=tk: B.index_reindex(ia, self.pool, tk, self.iws, stream)))
            if self._swa_new[l]:
                out.append(("quantize_window", lambda l=l: self.quantize_window(l, stream)))
            out.append(("attention", lambda l=l: B.sparse_attn(self.aargs[l], self.aws, stream)))
        return out

    # one pass of the whole layer sequence
    def step(self, stream=None) -> None:
        for _, call in self.calls(stream):
            call()
