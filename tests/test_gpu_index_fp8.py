"""GPU parity of the real-valued (FP8) indexer against the oracle
(oracle.indexer_fp8, FP64).

The library evaluates FP8 scores in fp32, so they are compared with the
oracle's exact scores within the rounding bound of tests.parity
(fp8_score_bound): every visible position's score (decoded from the scan's
workspace keys), and the pool and Top-512 rows, each of which must be a valid
selection for some scores within that bound.  Where the scores are exact in
fp32 (small integers in E4M3 codes, unit scales) the result must equal the
integer indexer's bit for bit."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e4m3_amd as csa2
from fp4_kv_cache_e4m3_amd import synth
from oracle import indexer as oidx
from oracle import indexer_fp8 as o8
from tests.parity import dev, fp8_full_errors, fp8_score_bound, fp8_topk_errors, host, keys_to_scores

pytestmark = pytest.mark.gpu


def finite_codes(rng, size):
    """E4M3FN codes over every finite value: zeros of both signs, subnormals, 448."""
    c = rng.integers(0, 254, size=size).astype(np.uint8)
    c[c >= 0x7F] += 1
    return c


def synth_like_codes(rng, size):
    v = rng.integers(0, 96, size=size).astype(np.uint8)
    return np.where(v < 48, v + 0x28, (v - 48 + 0x28) | 0x80).astype(np.uint8)


def inputs(seed, B, Qn, T, HI, DI, kind):
    rng = np.random.default_rng(seed)
    codes = finite_codes if kind == "all" else synth_like_codes
    cq = codes(rng, (B * Qn, HI, DI))
    ck = codes(rng, (B, T, DI))
    sq = ((rng.random((B * Qn, HI)) + 1.0) / 32).astype(np.float32)
    sk = ((rng.random((B, T)) + 1.0) / 32).astype(np.float32)
    iw = (rng.random((B * Qn, HI)) * 1.25 - 0.25).astype(np.float32)
    return cq, sq, iw, ck, sk


# from 2^19 positions on, the scan writes block maxima only (no token keys)
LONG_T = 1 << 19


def run_full(cq, sq, iw, ck, sk, qn, n_visible=None):
    """Scan and select as two calls: (pool, topk, token scores [nq, T] decoded
    from the scan's workspace keys, NaN where no key was written; None for
    contexts of LONG_T positions or more)."""
    d = [dev(a) for a in (cq, sq, iw, ck, sk)]
    nv_d = dev(np.asarray(n_visible, dtype=np.int32)) if n_visible is not None else None
    nq, T = cq.shape[0], ck.shape[1]
    pool = torch.full((nq, 2048), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((nq, 512), -7, dtype=torch.int32, device="cuda")
    args = csa2.index_args(d[0], d[2], d[3], qn, nv_d, q_scale=d[1], k_scale=d[4])
    assert args.fp8 == 1
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    csa2.index_scan(args, ws)
    scores = None
    if T < LONG_T:                      # the scan's token keys are in the workspace
        tk_stride = (T + 15) // 16 * 16
        keys = host(ws)[: nq * tk_stride * 4].view(np.uint32).reshape(nq, tk_stride)[:, :T]
        scores = keys_to_scores(keys)
    csa2.index_select(args, pool, topk, ws)
    return host(pool), host(topk), scores


def run_reindex(cq, sq, iw, ck, sk, qn, pool, n_visible=None):
    d = [dev(a) for a in (cq, sq, iw, ck, sk)]
    nv_d = dev(np.asarray(n_visible, dtype=np.int32)) if n_visible is not None else None
    topk = torch.full((cq.shape[0], 512), -7, dtype=torch.int32, device="cuda")
    args = csa2.index_args(d[0], d[2], d[3], qn, nv_d, q_scale=d[1], k_scale=d[4])
    ws = torch.empty(max(256, csa2.index_workspace_size(args)), dtype=torch.uint8, device="cuda")
    csa2.index_reindex(args, dev(pool.astype(np.int32)), topk, ws)
    return host(topk)


def check_full(cq, sq, iw, ck, sk, qn, pool, topk, scores, n_visible=None):
    """Scores within the bound, pool and Top-512 valid; returns the number of
    queries whose rows equal the oracle's exactly."""
    nq, HI, DI = cq.shape
    T = ck.shape[1]
    rpool, rtopk = o8.index_full(cq, sq, iw, ck, sk, qn, n_visible)
    exact = 0
    for q in range(nq):
        b = q // qn
        nv = T if n_visible is None else int(n_visible[q])
        s = o8.token_scores(cq[q], sq[q], iw[q], ck[b, :nv], sk[b, :nv])
        eps = fp8_score_bound(o8.abs_scores(cq[q], sq[q], iw[q], ck[b, :nv], sk[b, :nv]), DI, HI)
        if scores is not None:
            err = np.abs(scores[q, :nv] - s)
            assert np.all(err <= eps), f"query {q}: score off by {float((err - eps).max())} beyond the bound"
        problems = fp8_full_errors(pool[q], topk[q], s, eps, nv)
        assert problems == [], f"query {q}: {problems}"
        exact += int(np.array_equal(pool[q], rpool[q]) and np.array_equal(topk[q], rtopk[q]))
    return exact


CASES = [  # (B, Qn, T, H_I, D_I, kind)
    (1, 1, 1, 2, 64, "all"),
    (2, 1, 9, 8, 128, "all"),
    (1, 1, 4096, 2, 64, "synth"),
    (3, 1, 5003, 8, 128, "all"),
    (2, 6, 20011, 8, 128, "synth"),     # several queries per sequence, pool drops blocks
    (2, 4, 17003, 16, 64, "all"),
    (1, 3, 33000, 4, 128, "synth"),
    (1, 2, 100003, 8, 128, "synth"),    # more than 8,192 blocks
    (2, 1, 2500, 2, 64, "all"),         # fewer than 512 blocks
    (1, 16, 9000, 8, 128, "synth"),     # 128 score rows: two scan workgroups per key chunk
    (2, 9, 12000, 16, 64, "all"),       # 144 score rows: three, the last partial
    (1, 3, 600001, 8, 128, "synth"),    # long context: Top-512 from the rescored pool
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}Q{}T{}H{}D{}{}".format(*c))
def test_index_full_fp8_matches_oracle(case):
    B, Qn, T, HI, DI, kind = case
    cq, sq, iw, ck, sk = inputs(sum(case[:5]), B, Qn, T, HI, DI, kind)
    pool, topk, scores = run_full(cq, sq, iw, ck, sk, Qn)
    exact = check_full(cq, sq, iw, ck, sk, Qn, pool, topk, scores)
    assert exact >= (B * Qn + 1) // 2


def test_index_full_fp8_n_visible_ragged():
    B, Qn, T = 2, 3, 20000
    cq, sq, iw, ck, sk = inputs(11, B, Qn, T, 8, 128, "all")
    nv = np.array([T, 0, 1, 16385, 7, 12345], dtype=np.int32)
    pool, topk, scores = run_full(cq, sq, iw, ck, sk, Qn, nv)
    check_full(cq, sq, iw, ck, sk, Qn, pool, topk, scores, nv)
    assert np.all(pool[1] == -1) and np.all(topk[1] == -1)


def test_index_fp8_integer_codes_equal_integer_indexer():
    """Small integers in E4M3 codes with unit scales: every fp32 score is
    exact, so pool and Top-512 equal the integer indexer's bit for bit."""
    rng = np.random.default_rng(21)
    B, Qn, T, HI, DI = 2, 2, 30011, 8, 128
    iq = rng.integers(-8, 9, size=(B * Qn, HI, DI))
    ik = rng.integers(-8, 9, size=(B, T, DI))
    iw = rng.integers(1, 9, size=(B * Qn, HI)).astype(np.float32)
    to_codes = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    cq, ck = to_codes(iq), to_codes(ik)
    sq = np.ones((B * Qn, HI), np.float32)
    sk = np.ones((B, T), np.float32)
    pool, topk, _ = run_full(cq, sq, iw, ck, sk, Qn)
    rpool, rtopk = oidx.index_full(iq.astype(np.int8), iw, ik.astype(np.int8), Qn)
    np.testing.assert_array_equal(pool, rpool)
    np.testing.assert_array_equal(topk, rtopk)
    np.testing.assert_array_equal(run_reindex(cq, sq, iw, ck, sk, Qn, rpool),
                                  oidx.index_reindex(iq.astype(np.int8), iw, ik.astype(np.int8), Qn, rpool))


REINDEX_CASES = [(3, 1, 5003, 8, 128, "all"), (2, 6, 20011, 8, 128, "synth"), (2, 4, 17003, 16, 64, "all"),
                 (1, 1, 2000, 2, 64, "synth")]


@pytest.mark.parametrize("case", REINDEX_CASES, ids=lambda c: "B{}Q{}T{}H{}D{}{}".format(*c))
def test_index_reindex_fp8_matches_oracle(case):
    B, Qn, T, HI, DI, kind = case
    cq0, sq0, iw0, ck, sk = inputs(sum(case[:5]), B, Qn, T, HI, DI, kind)
    rpool, _ = o8.index_full(cq0, sq0, iw0, ck, sk, Qn)            # the Full layer's pool (oracle)
    cq, sq, iw, _, _ = inputs(sum(case[:5]) + 1000, B, Qn, 8, HI, DI, kind)
    topk = run_reindex(cq, sq, iw, ck, sk, Qn, rpool)
    rtopk = o8.index_reindex(cq, sq, iw, ck, sk, Qn, rpool)
    exact = 0
    for q in range(B * Qn):
        b = q // Qn
        _, cand, s = o8.reindex_query(cq[q], sq[q], iw[q], ck[b], sk[b], rpool[q], T)
        eps = fp8_score_bound(o8.abs_scores(cq[q], sq[q], iw[q], ck[b, cand], sk[b, cand]), DI, HI)
        problems = fp8_topk_errors(topk[q], cand, s, eps)
        assert problems == [], f"query {q}: {problems}"
        exact += int(np.array_equal(topk[q], rtopk[q]))
    assert exact >= (B * Qn + 1) // 2


@pytest.fixture(scope="module")
def idx8_inputs():
    w = synth.C2_IDX8
    ck = synth.index_k_all(w)
    sk = synth.index_k_scale_all(w)
    return w, ck, sk


def test_index_full_fp8_batch32_t65536(idx8_inputs):
    w, ck, sk = idx8_inputs
    cq, sq, iw = synth.index_q(w), synth.index_q_scale(w), synth.index_w(w)
    pool, topk, scores = run_full(cq, sq, iw, ck, sk, 1)
    exact = check_full(cq, sq, iw, ck, sk, 1, pool, topk, scores)
    assert exact >= 24, f"only {exact} of 32 queries equal the oracle's selection"
    pool2, topk2, scores2 = run_full(cq, sq, iw, ck, sk, 1)          # deterministic
    np.testing.assert_array_equal(pool, pool2)
    np.testing.assert_array_equal(topk, topk2)
    np.testing.assert_array_equal(scores, scores2)


def test_index_reindex_fp8_batch32_t65536(idx8_inputs):
    w, ck, sk = idx8_inputs
    rpool, _ = o8.index_full(synth.index_q(w, 0, pool_source=True), synth.index_q_scale(w, 0, pool_source=True),
                             synth.index_w(w, 0, pool_source=True), ck, sk, 1)
    cq, sq, iw = synth.index_q(w, 1), synth.index_q_scale(w, 1), synth.index_w(w, 1)
    topk = run_reindex(cq, sq, iw, ck, sk, 1, rpool)
    rtopk = o8.index_reindex(cq, sq, iw, ck, sk, 1, rpool)
    exact = 0
    for q in range(w.nq):
        _, cand, s = o8.reindex_query(cq[q], sq[q], iw[q], ck[q], sk[q], rpool[q], w.kv_len)
        eps = fp8_score_bound(o8.abs_scores(cq[q], sq[q], iw[q], ck[q, cand], sk[q, cand]), w.idx_dim, w.idx_heads)
        problems = fp8_topk_errors(topk[q], cand, s, eps)
        assert problems == [], f"query {q}: {problems}"
        exact += int(np.array_equal(topk[q], rtopk[q]))
    assert exact >= 24
