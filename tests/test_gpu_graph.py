"""A whole decode-group step captured in a HIP graph (torch.cuda.CUDAGraph):
every library call enqueues kernels only (no allocation, no host sync, no
memset node), so replays must reproduce the eager step bit for bit.  The
outputs (and, with 8-bit windows, the new window rows the attention calls
store) are clobbered eagerly before each replay, and eager work and
synchronisations run between the replays."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_e4m3_amd import DecodeGroup, synth
from tests.parity import host

pytestmark = pytest.mark.gpu


def snapshot(g):
    T, n = g.w.kv_len, g.w.new_per_seq
    new_rows = torch.from_numpy(np.concatenate([g.cache_rows(b, np.arange(T - n, T)) for b in range(g.w.batch)]))
    new_rows = new_rows.to(g.codes.device)
    win = []
    if g.w.swa8:                                          # the 8-bit windows the attention calls write into
        for l in range(len(g.w.layers)):
            win += [host(g.swa[l]), host(g.swa_scale[l])]
    return ([host(o) for o in g.out] + [host(t) for t in g.topks] + [host(g.pool)]
            + [host(g.codes[new_rows]), host(g.scales[new_rows])] + win)


def clobber(g):
    for o in g.out:
        o.fill_(float("nan"))
    for t in g.topks:
        t.fill_(-7)
    if "full" in g.w.layers:                              # otherwise the pool is an input
        g.pool.fill_(-7)
    if g.w.swa8:                                          # the step's new window rows' slots
        R, Qn = g.w.swa_rows, g.w.q_per_seq
        for l in range(len(g.w.layers)):
            g.swa[l][:, R - Qn:].fill_(0xA5)
            g.swa_scale[l][:, R - Qn:].fill_(float("nan"))


@pytest.mark.parametrize("name", ["decode_group_full_reuse3_b32_t65536", "decode_group_reindex_reuse3_b32_t65536",
                                  "decode_group_full_reuse3_b32_t65536_paged",
                                  "decode_group_full_reuse3_b32_t65536_swa8"])
def test_step_graph_replays_match_eager(name):
    w = synth.WORKLOADS[name]
    g = DecodeGroup(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                        # eager warm-up on the capture stream
        g.step(side)
    torch.cuda.synchronize()
    ref = snapshot(g)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        g.step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        clobber(g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(g)
        for i, (a, b) in enumerate(zip(got, ref)):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}, buffer {i}")
        g.step()                                          # eager work between replays
        torch.cuda.synchronize()
