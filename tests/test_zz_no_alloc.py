"""csa2_index_full_noalloc (the Full-layer index call on the library's fixed
per-GPU scratch, for callers that cannot allocate) against csa2_index_full
with a caller workspace: pool and Top-512 bit-identical, on two calls in a
row whose second is smaller (the scratch keeps the first call's keys), and a
host-side rejection of sizes past the scratch."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from tests.parity import dev, host

pytestmark = pytest.mark.gpu


def index_inputs(seed, B, Qn, T, HI=8, DI=128):
    rng = np.random.default_rng(seed)
    iq = rng.integers(-8, 9, size=(B * Qn, HI, DI), dtype=np.int8)
    iw = rng.integers(1, 9, size=(B * Qn, HI)).astype(np.float32)
    ik = rng.integers(-8, 9, size=(B, T, DI), dtype=np.int8)
    return [dev(a) for a in (iq, iw, ik)]


def both(seed, B, Qn, T):
    iq, iw, ik = index_inputs(seed, B, Qn, T)
    args = csa2.index_args(iq, iw, ik, Qn)
    nq = B * Qn
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    ref_pool = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    ref_topk = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
    csa2.index_full(args, ref_pool, ref_topk, ws)
    pool = torch.full((nq, 2048), -9, dtype=torch.int32, device="cuda")
    topk = torch.full((nq, 512), -9, dtype=torch.int32, device="cuda")
    csa2.index_full_noalloc(args, pool, topk)
    return host(pool), host(topk), host(ref_pool), host(ref_topk)


def test_noalloc_equals_workspace_call_twice():
    # first call: 2 queries over 2^19 positions (block maxima only), then 16
    # sequences x 40,000 positions (token keys), then a smaller and ragged one,
    # all over the same scratch
    for seed, (B, Qn, T) in [(4, (1, 2, 1 << 19)), (1, (16, 1, 40000)), (2, (3, 2, 5003))]:
        pool, topk, rpool, rtopk = both(seed, B, Qn, T)
        np.testing.assert_array_equal(pool, rpool)
        np.testing.assert_array_equal(topk, rtopk)
        assert (topk >= 0).sum() == B * Qn * 512


def test_noalloc_rejects_sizes_past_the_scratch():
    iq, iw, ik = index_inputs(3, 1, 1, 16)
    # 256 query rows over 2^20 positions need 256 x 2^17 x 4 B of block keys
    # and 256 x 2,048 x 4 B of pool: more than 64 MiB
    big = csa2.IndexArgs(256, 1, 1 << 20, 8, 128, iq.data_ptr(), iw.data_ptr(), ik.data_ptr(), None)
    assert csa2.index_workspace_size(big) > (64 << 20)
    st = csa2.load().csa2_index_full_noalloc(big, None, 16, None)
    assert st == 6
    assert "scratch" in csa2.status_string(st)
