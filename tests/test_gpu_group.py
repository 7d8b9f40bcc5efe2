"""End-to-end parity of one layer-group step (the sequence bench.py times):
quantise the step's new entries, index (Full or Reindex), then attention for
every layer of the group -- all through the C ABI, compared with the oracle run
on the same seeded inputs (on every query, or on a sample of them for the
large prefill and 1M-entry groups)."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_e4m3_amd import DecodeGroup, synth
from oracle import indexer as oidx
from tests.parity import ATTN_TOL, host, oracle_attention, oracle_kv_rows, oracle_selected_rows, rownorm_err

pytestmark = pytest.mark.gpu


def _pad(ids, width):
    out = np.full(width, -1, dtype=np.int32)
    out[:len(ids)] = ids
    return out


def check_group(w, sample=None):
    g = DecodeGroup(w)
    g.step()
    torch.cuda.synchronize()
    qs = list(range(w.nq)) if sample is None else list(sample)
    seqs = sorted({q // w.q_per_seq for q in qs})
    T = w.kv_len
    ik = {b: synth.index_k(w, b) for b in seqs}
    rtopk = np.full((w.nq, 512), -1, dtype=np.int32)
    got_pool, got_topk = host(g.pool), host(g.topk)
    if w.layers[0] == "full":
        iq, iw = synth.index_q(w), synth.index_w(w)
        for q in qs:
            pool, topk, _ = oidx.full_query(iq[q], iw[q], ik[q // w.q_per_seq], T)
            rtopk[q] = _pad(topk, 512)
            if not w.encoder:
                np.testing.assert_array_equal(got_pool[q], _pad(pool, 2048))
    else:
        iq0, iw0 = synth.index_q(w, 0, pool_source=True), synth.index_w(w, 0, pool_source=True)
        iq, iw = synth.index_q(w), synth.index_w(w)
        for q in qs:
            pool, _, _ = oidx.full_query(iq0[q], iw0[q], ik[q // w.q_per_seq], T)
            np.testing.assert_array_equal(got_pool[q], _pad(pool, 2048))
            rtopk[q] = _pad(oidx.reindex_query(iq[q], iw[q], ik[q // w.q_per_seq], pool, T), 512)
    del ik
    np.testing.assert_array_equal(got_topk[qs], rtopk[qs])
    if w.layers[0] == "full":            # the step's new FP4 rows (Full layers write their KV)
        n = w.new_per_seq
        for b in (0, w.batch - 1):
            rc, rs = oracle_kv_rows(w, b, np.arange(T - n, T), with_new_rows=True)
            np.testing.assert_array_equal(host(g.codes[b * T + T - n:b * T + T]), rc)
            np.testing.assert_array_equal(host(g.scales[b * T + T - n:b * T + T]), rs)
    # every layer of the group attends over the same Top-K rows
    rows = oracle_selected_rows(w, rtopk, qs, with_new_rows=(w.layers[0] == "full"))
    for l in range(len(w.layers)):
        got = host(g.out[l])
        ref = oracle_attention(w, synth.attn_q_bf16(w, l), synth.swa_bf16(w, l), rtopk,
                               with_new_rows=(w.layers[0] == "full"), queries=qs, rows=rows)
        err = rownorm_err(got[qs], ref[qs])
        assert err <= ATTN_TOL, (l, err)


def test_group_full_decode_t4096():
    check_group(synth.C1.replace(layers=("full", "reuse")))


def test_group_full_reuse3_batch32_t65536():
    check_group(synth.C2)


def test_group_reindex_reuse3_batch32_t65536():
    check_group(synth.C3, sample=range(0, 32, 3))


def test_group_prefill_q4096_t65536():
    """Encoder group: 4,096 query tokens over 65,536 entries, Full + 5 Reuse,
    2,048 new entries quantised; sampled queries across the chunk."""
    check_group(synth.C4, sample=[0, 1, 127, 128, 1000, 2047, 3333, 4095])


def test_group_verify_b8_q6_t1m():
    """1M-entry verify group: 8 sequences x (1 + 5 draft) queries, 6 new
    entries per sequence; the first and the last sequence are checked."""
    w = synth.C5
    check_group(w, sample=list(range(6)) + list(range(w.nq - 6, w.nq)))
