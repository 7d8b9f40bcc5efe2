"""A whole decode-group step captured in a HIP graph (torch.cuda.CUDAGraph):
every library call enqueues kernels only (no allocation, no host sync, no
memset node), so replays must reproduce the eager step bit for bit.  The
outputs are clobbered eagerly before each replay, and eager work and
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
    return ([host(o) for o in g.out] + [host(t) for t in g.topks] + [host(g.pool)]
            + [host(g.codes[new_rows]), host(g.scales[new_rows])])


def clobber(g):
    for o in g.out:
        o.fill_(float("nan"))
    for t in g.topks:
        t.fill_(-7)
    if "full" in g.w.layers:                              # otherwise the pool is an input
        g.pool.fill_(-7)


@pytest.mark.parametrize("name", ["decode_group_full_reuse3_b32_t65536", "decode_group_reindex_reuse3_b32_t65536",
                                  "decode_group_full_reuse3_b32_t65536_paged"])
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
