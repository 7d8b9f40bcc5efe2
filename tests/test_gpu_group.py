"""End-to-end parity of one layer-group step (the sequence bench.py times):
quantise the new tokens, index (Full or Reindex), then attention for every
layer of the group -- all through the C ABI, compared with the oracle run on
the same seeded inputs."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_e4m3_amd import DecodeGroup, synth
from oracle import indexer as oidx
from tests.parity import ATTN_TOL, host, oracle_attention, oracle_kv_rows, rownorm_err

pytestmark = pytest.mark.gpu


def check_group(w, sample_queries=None):
    g = DecodeGroup(w)
    g.step()
    torch.cuda.synchronize()
    ik = synth.index_k_all(w)
    if w.layers[0] == "full":
        iq, iw = synth.index_q(w), synth.index_w(w)
        rpool, rtopk = oidx.index_full(iq, iw, ik, w.q_per_seq)
        np.testing.assert_array_equal(host(g.pool), rpool)
    else:
        iq0, iw0 = synth.index_q(w, 0, pool_source=True), synth.index_w(w, 0, pool_source=True)
        rpool, _ = oidx.index_full(iq0, iw0, ik, w.q_per_seq)
        np.testing.assert_array_equal(host(g.pool), rpool)
        rtopk = oidx.index_reindex(synth.index_q(w), synth.index_w(w), ik, w.q_per_seq, rpool)
    del ik
    np.testing.assert_array_equal(host(g.topk), rtopk)
    T = w.kv_len
    if w.layers[0] == "full":            # the new tokens' FP4 rows (Full layers write their KV)
        for b in (0, w.batch - 1):
            rc, rs = oracle_kv_rows(w, b, np.array([T - 1]), with_new_rows=True)
            np.testing.assert_array_equal(host(g.codes[b * T + T - 1:b * T + T]), rc)
            np.testing.assert_array_equal(host(g.scales[b * T + T - 1:b * T + T]), rs)
    for l in range(len(w.layers)):
        got = host(g.out[l])
        ref = oracle_attention(w, synth.attn_q_bf16(w, l), synth.swa_bf16(w, l), rtopk,
                               with_new_rows=(w.layers[0] == "full"), queries=sample_queries)
        sel = slice(None) if sample_queries is None else list(sample_queries)
        err = rownorm_err(got[sel], ref[sel])
        assert err <= ATTN_TOL, (l, err)


def test_group_full_decode_t4096():
    check_group(synth.C1.replace(layers=("full", "reuse")))


def test_group_full_reuse3_batch32_t65536():
    check_group(synth.C2)


def test_group_reindex_reuse3_batch32_t65536():
    check_group(synth.C3, sample_queries=range(0, 32, 3))
