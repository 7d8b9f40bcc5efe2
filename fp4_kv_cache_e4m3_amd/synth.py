"""Seeded synthetic inputs for the CSA2 hot path (shared by tests, smoke and bench).

This module only *draws* inputs: shapes, value distributions and seeds.  It
holds none of the method's arithmetic (no quantisation, scoring, selection or
attention), so both the HIP path and the oracle can consume what it produces.

Workloads mirror the shapes of the CSA2 decode/prefill path described on the
DeepSeek-V4.1-Flash pages (ai-maestro.online, section "Compressed Sparse
Attention 2": Top-512, 2,048 blocks x 8 tokens, 128-token sliding window; FP4
main KV with one E4M3 scale per 16 channels, section "FP4 KV, Bounded Replay,
and other extensions").  Because the pages publish no activations, every
tensor is drawn from a fixed distribution:

* main-KV source rows: fp32 N(0, 1), later quantised to FP4;
* indexer q / k: integers uniform in [-r, r] (int8), head weights integers
  uniform in [1, w_max] stored as fp32 -- so every indexer score is an exact
  integer in fp32;
* attention Q and SWA rows: N(0, 1) rounded to bf16 (round-to-nearest-even);
* FP8 indexer (``idx_fp8``): q / k bytes are E4M3FN codes drawn uniformly
  over the 96 codes of magnitude [0.25, 15] and either sign (a log-uniform
  spread over six octaves), key scales one per position and query scales one
  per (query, head), fp32 uniform in [1/32, 1/16), head weights fp32 uniform
  in [-0.25, 1).

Seeds: ``SeedSequence([0xC5A2, workload_id, tensor_id, layer, chunk])``.
Large tensors are drawn in fixed-size row chunks so any chunk can be redrawn
on its own.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 0xC5A2

# tensor ids used in the seed tuple
T_KV_SRC = 1      # fp32 source rows of the main KV cache
T_IK = 2          # indexer keys, int8
T_IQ = 3          # indexer queries, int8 (per layer)
T_IW = 4          # indexer head weights (per layer)
T_Q = 5           # attention queries, bf16 (per layer)
T_SWA = 6         # sliding-window rows, bf16 (per layer)
T_NEW = 7         # fp32 rows of the tokens appended this step
T_IQ_POOL = 8     # indexer q of the Full layer that produced a Reindex pool
T_IW_POOL = 9
T_IK_SCALE = 10   # fp32 per-position scales of FP8 indexer keys
T_IQ_SCALE = 11   # fp32 per-(query, head) scales of FP8 indexer queries (per layer)
T_IQ_SCALE_POOL = 12
T_PAGES = 13      # page order of a paged cache
T_RING = 14       # window ring start slots
T_NEW_SWA = 15    # bf16 window rows of the tokens appended this step (per layer)

# FP8 indexer codes: magnitude codes 0x28..0x57 (E4M3 values 0.25 .. 15), either sign
_E4M3_LO, _E4M3_N = 0x28, 48

KV_CHUNK_ROWS = 4096   # rows per independently seeded chunk of the KV source / ik


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic CSA2 workload."""

    name: str
    wid: int                 # id folded into every seed
    batch: int               # B sequences
    q_per_seq: int           # Qn query tokens per sequence (1 for decode)
    kv_len: int              # T compressed main-KV entries per sequence
    dim: int                 # d, main KV / Q / SWA row width
    heads: int               # H attention heads
    window: int              # W sliding-window rows per query
    idx_heads: int           # H_I indexer heads
    idx_dim: int             # D_I indexer dim
    idx_range: int           # indexer q/k integers uniform in [-r, r]
    w_max: int               # indexer head weights integers uniform in [1, w_max]
    layers: tuple = ("full",)  # CSA2 layer modes of the group
    ratio: int = 1           # tokens per compressed entry
    encoder: bool = False    # encoder (prefill) group: no Reindex layer consumes the pool
    swa8: bool = False       # window rows kept as 8-bit codes (quantised from the same bf16 rows)
    idx_fp8: bool = False    # indexer q / k as E4M3 codes with fp32 scales instead of integers
    page_size: int = 0       # > 0: the FP4 cache is paged (pages of this many rows, shuffled)
    swa_ring: bool = False   # window rows held in a ring buffer with a per-sequence start slot
    note: str = ""

    @property
    def nq(self) -> int:
        return self.batch * self.q_per_seq

    @property
    def swa_rows(self) -> int:
        return self.window - 1 + self.q_per_seq

    @property
    def new_per_seq(self) -> int:
        """Main-KV entries a step appends per sequence (its query tokens / ratio)."""
        return max(1, self.q_per_seq // self.ratio)

    def replace(self, **kw) -> "Workload":
        d = {f: getattr(self, f) for f in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


# The five workloads (shapes and distributions of the pages' decode/prefill path).
C1 = Workload("full_decode_t4096_d128", 1, batch=1, q_per_seq=1, kv_len=4096, dim=128,
              heads=8, window=128, idx_heads=2, idx_dim=64, idx_range=4, w_max=4,
              layers=("full",), note="one Full layer decode step, single sequence")
C2 = Workload("decode_group_full_reuse3_b32_t65536", 2, batch=32, q_per_seq=1, kv_len=65536,
              dim=512, heads=64, window=128, idx_heads=8, idx_dim=128, idx_range=8, w_max=8,
              layers=("full", "reuse", "reuse", "reuse"),
              note="decoder group 1: Full + 3 Reuse, batch 32, 64K entries")
C3 = Workload("decode_group_reindex_reuse3_b32_t65536", 3, batch=32, q_per_seq=1, kv_len=65536,
              dim=512, heads=64, window=128, idx_heads=8, idx_dim=128, idx_range=8, w_max=8,
              layers=("reindex", "reuse", "reuse", "reuse"),
              note="decoder groups 2-5: Reindex + 3 Reuse")
C4 = Workload("prefill_group_full_reuse5_q4096_t65536", 4, batch=1, q_per_seq=4096, kv_len=65536,
              dim=512, heads=64, window=128, idx_heads=8, idx_dim=128, idx_range=8, w_max=8,
              layers=("full",) + ("reuse",) * 5, ratio=2, encoder=True,
              note="encoder prefill chunk, 4096 queries over 65536 compressed entries")
C5 = Workload("verify_group_full_reuse3_b8_q6_t1m", 5, batch=8, q_per_seq=6, kv_len=1 << 20,
              dim=512, heads=64, window=128, idx_heads=8, idx_dim=128, idx_range=8, w_max=8,
              layers=("full", "reuse", "reuse", "reuse"),
              note="1M-entry decode with 1 + 5 draft queries per sequence")

# The whole decoder at decode: group 1 (Full + 3 Reuse) followed by four
# Reindex + 3 Reuse groups, each Reindex layer rescoring the pool of the Full
# layer of the same step (20 layers).
C6 = Workload("decoder_step_full_reindex4_b32_t65536", 6, batch=32, q_per_seq=1, kv_len=65536,
              dim=512, heads=64, window=128, idx_heads=8, idx_dim=128, idx_range=8, w_max=8,
              layers=("full", "reuse", "reuse", "reuse") + ("reindex", "reuse", "reuse", "reuse") * 4,
              note="20-layer decoder step: Full group + 4 Reindex groups, batch 32, 64K entries")

# decoder group 1 with the sliding window kept in 8 bits (same seeds as C2)
C2_SWA8 = C2.replace(name="decode_group_full_reuse3_b32_t65536_swa8", swa8=True,
                     note="decoder group 1 with 8-bit (E4M3 + row scale) window rows")

# decoder group 1 with a real-valued (E4M3 + fp32 scales) indexer
C2_IDX8 = C2.replace(name="decode_group_full_reuse3_b32_t65536_idx8", wid=8, idx_fp8=True,
                     note="decoder group 1 with FP8 indexer keys and queries")

# decoder group 1 over a paged FP4 cache (256-row pages in shuffled order)
# and ring-buffer windows
C2_PAGED = C2.replace(name="decode_group_full_reuse3_b32_t65536_paged", wid=9, page_size=256, swa_ring=True,
                      note="decoder group 1 over a paged FP4 cache and ring-buffer windows")

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5, C6, C2_SWA8, C2_IDX8, C2_PAGED)}


def _rng(w: Workload, tensor: int, layer: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, w.wid, tensor, layer, chunk]))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bit patterns.

    Used only to *draw* bf16 inputs.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- generators
def kv_source_rows(w: Workload, b: int, row0: int, nrows: int, layer: int = 0) -> np.ndarray:
    """fp32 N(0,1) source rows [row0, row0+nrows) of sequence b's main KV (before FP4)."""
    out = np.empty((nrows, w.dim), dtype=np.float32)
    c0 = row0 // KV_CHUNK_ROWS
    c1 = (row0 + nrows - 1) // KV_CHUNK_ROWS if nrows else c0 - 1

    def one(c):
        rows = min(KV_CHUNK_ROWS, w.kv_len - c * KV_CHUNK_ROWS)
        g = _rng(w, T_KV_SRC, layer, b * 100003 + c)
        chunk = g.standard_normal((rows, w.dim), dtype=np.float32)
        lo = max(row0, c * KV_CHUNK_ROWS)
        hi = min(row0 + nrows, c * KV_CHUNK_ROWS + rows)
        out[lo - row0:hi - row0] = chunk[lo - c * KV_CHUNK_ROWS:hi - c * KV_CHUNK_ROWS]

    chunks = list(range(c0, c1 + 1))
    if len(chunks) > 2:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, chunks))
    else:
        for c in chunks:
            one(c)
    return out


def kv_source(w: Workload, b: int, layer: int = 0) -> np.ndarray:
    return kv_source_rows(w, b, 0, w.kv_len, layer)


def new_rows(w: Workload, step: int = 0) -> np.ndarray:
    """fp32 N(0,1) rows of the main-KV entries one step appends,
    [B * new_per_seq, d]; row b * new_per_seq + i lands in slot
    T - new_per_seq + i of sequence b."""
    return _rng(w, T_NEW, step).standard_normal((w.batch * w.new_per_seq, w.dim), dtype=np.float32)


def _e4m3_codes(g: np.random.Generator, size) -> np.ndarray:
    v = g.integers(0, 2 * _E4M3_N, size=size, dtype=np.uint8)
    return np.where(v < _E4M3_N, v + _E4M3_LO, (v - _E4M3_N + _E4M3_LO) | 0x80).astype(np.uint8)


def _fp8_scales(g: np.random.Generator, size) -> np.ndarray:
    return ((g.random(size, dtype=np.float32) + np.float32(1.0)) * np.float32(1.0 / 32)).astype(np.float32)


def index_k_rows(w: Workload, b: int, row0: int, nrows: int) -> np.ndarray:
    """Indexer keys of sequence b, rows [row0, row0+nrows): int8 in [-r, r], or
    uint8 E4M3 codes for an FP8 indexer."""
    out = np.empty((nrows, w.idx_dim), dtype=np.uint8 if w.idx_fp8 else np.int8)
    c0 = row0 // KV_CHUNK_ROWS
    c1 = (row0 + nrows - 1) // KV_CHUNK_ROWS if nrows else c0 - 1
    for c in range(c0, c1 + 1):
        rows = min(KV_CHUNK_ROWS, w.kv_len - c * KV_CHUNK_ROWS)
        g = _rng(w, T_IK, 0, b * 100003 + c)
        if w.idx_fp8:
            chunk = _e4m3_codes(g, (rows, w.idx_dim))
        else:
            chunk = g.integers(-w.idx_range, w.idx_range + 1, size=(rows, w.idx_dim), dtype=np.int8)
        lo = max(row0, c * KV_CHUNK_ROWS)
        hi = min(row0 + nrows, c * KV_CHUNK_ROWS + rows)
        out[lo - row0:hi - row0] = chunk[lo - c * KV_CHUNK_ROWS:hi - c * KV_CHUNK_ROWS]
    return out


def index_k(w: Workload, b: int) -> np.ndarray:
    return index_k_rows(w, b, 0, w.kv_len)


def index_k_scale(w: Workload, b: int) -> np.ndarray:
    """[T] fp32 per-position scales of sequence b's FP8 indexer keys."""
    return _fp8_scales(_rng(w, T_IK_SCALE, 0, b), w.kv_len)


def index_k_scale_all(w: Workload) -> np.ndarray:
    """[B, T] fp32."""
    return np.stack([index_k_scale(w, b) for b in range(w.batch)])


def index_k_all(w: Workload) -> np.ndarray:
    """[B, T, D_I] int8 (uint8 E4M3 codes for an FP8 indexer)."""
    out = np.empty((w.batch, w.kv_len, w.idx_dim), dtype=np.uint8 if w.idx_fp8 else np.int8)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda b: out.__setitem__(b, index_k(w, b)), range(w.batch)))
    return out


def index_q(w: Workload, layer: int = 0, pool_source: bool = False) -> np.ndarray:
    """[nq, H_I, D_I] indexer queries of one layer: int8, or uint8 E4M3 codes."""
    t = T_IQ_POOL if pool_source else T_IQ
    g = _rng(w, t, layer)
    if w.idx_fp8:
        return _e4m3_codes(g, (w.nq, w.idx_heads, w.idx_dim))
    return g.integers(-w.idx_range, w.idx_range + 1, size=(w.nq, w.idx_heads, w.idx_dim), dtype=np.int8)


def index_q_scale(w: Workload, layer: int = 0, pool_source: bool = False) -> np.ndarray:
    """[nq, H_I] fp32 scales of the FP8 indexer queries of one layer."""
    t = T_IQ_SCALE_POOL if pool_source else T_IQ_SCALE
    return _fp8_scales(_rng(w, t, layer), (w.nq, w.idx_heads))


def index_w(w: Workload, layer: int = 0, pool_source: bool = False) -> np.ndarray:
    """[nq, H_I] fp32 head weights: integers in [1, w_max], or uniform in
    [-0.25, 1) for an FP8 indexer."""
    t = T_IW_POOL if pool_source else T_IW
    g = _rng(w, t, layer)
    if w.idx_fp8:
        return (g.random((w.nq, w.idx_heads), dtype=np.float32) * np.float32(1.25) - np.float32(0.25)).astype(np.float32)
    return g.integers(1, w.w_max + 1, size=(w.nq, w.idx_heads)).astype(np.float32)


def new_swa_rows(w: Workload, layer: int = 0) -> np.ndarray:
    """[B * Qn, d] bf16 bit patterns of N(0,1) window rows of the step's query
    tokens (one per query, the newest rows of the window)."""
    x = _rng(w, T_NEW_SWA, layer).standard_normal((w.nq, w.dim), dtype=np.float32)
    return f32_to_bf16_bits(x)


def page_count(w: Workload) -> tuple:
    """(pages per sequence, physical pages) of a paged cache: one sequence's
    worth of spare pages that no block-table entry names."""
    per_seq = (w.kv_len + w.page_size - 1) // w.page_size
    return per_seq, (w.batch + 1) * per_seq


def block_table(w: Workload) -> np.ndarray:
    """[B, pages per sequence] int32: distinct physical pages in random order."""
    per_seq, n_phys = page_count(w)
    return _rng(w, T_PAGES).permutation(n_phys)[: w.batch * per_seq].astype(np.int32).reshape(w.batch, per_seq)


def swa_ring_start(w: Workload, layer: int = 0) -> np.ndarray:
    """[B] int32 ring slot of each sequence's first window row."""
    return _rng(w, T_RING, layer).integers(0, w.swa_rows, size=w.batch).astype(np.int32)


def attn_q_bf16(w: Workload, layer: int = 0) -> np.ndarray:
    """[nq, H, d] bf16 bit patterns of N(0,1) queries."""
    x = _rng(w, T_Q, layer).standard_normal((w.nq, w.heads, w.dim), dtype=np.float32)
    return f32_to_bf16_bits(x)


def swa_bf16(w: Workload, layer: int = 0) -> np.ndarray:
    """[B, W-1+Qn, d] bf16 bit patterns of N(0,1) sliding-window rows."""
    x = _rng(w, T_SWA, layer).standard_normal((w.batch, w.swa_rows, w.dim), dtype=np.float32)
    return f32_to_bf16_bits(x)


@dataclass
class Small:
    """Helper for ad-hoc small shapes in tests (not one of the named workloads)."""
    batch: int = 1
    q_per_seq: int = 1
    kv_len: int = 64
    dim: int = 128
    heads: int = 8
    window: int = 128
    idx_heads: int = 2
    idx_dim: int = 64
    idx_range: int = 4
    w_max: int = 4
    layers: tuple = field(default=("full",))

    def workload(self, wid: int = 99, name: str = "small") -> Workload:
        return Workload(name, wid, self.batch, self.q_per_seq, self.kv_len, self.dim, self.heads,
                        self.window, self.idx_heads, self.idx_dim, self.idx_range, self.w_max,
                        self.layers)
