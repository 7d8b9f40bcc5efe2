"""Pins of the oracle's FP8 (E4M3 + fp32 scales) indexer (CPU only).

* It reduces to the integer indexer (itself pinned against brute force) when
  the codes hold small integers and the scales are 1.
* Power-of-two scales give the integer scores times the scales, exactly.
* ReLU sign identities: s(k) + s(-k) and s(k) - s(-k) against the absolute
  and the linear form, with values decoded by torch's float8_e4m3fn.
* Exact-rational brute force on tiny inputs (all codes, subnormals included).
* The pool invariant I1 and the scale-invariance of the selection."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import indexer, indexer_fp8


def e4m3_codes_of(x: np.ndarray) -> np.ndarray:
    """E4M3FN codes of values that the format holds exactly (torch's cast)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back, np.asarray(x, dtype=np.float32))
    return t.view(torch.uint8).numpy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_codes(rng, size):
    """Random E4M3FN codes over every finite value (subnormals and zeros included)."""
    c = rng.integers(0, 254, size=size).astype(np.uint8)
    c[c >= 0x7F] += 1                                  # skip 0x7F (NaN); 0xFF is never drawn
    return c


def int_inputs(rng, nq, B, T, HI, DI, r, wmax):
    iq = rng.integers(-r, r + 1, size=(nq, HI, DI))
    iw = rng.integers(1, wmax + 1, size=(nq, HI)).astype(np.float32)
    ik = rng.integers(-r, r + 1, size=(B, T, DI))
    return iq, iw, ik


@pytest.mark.parametrize("T,HI,DI,r", [(1, 2, 8, 1), (9, 2, 8, 1), (513, 4, 16, 2), (1000, 8, 64, 8),
                                       (20000, 2, 4, 1)])
def test_reduces_to_integer_indexer(T, HI, DI, r):
    rng = np.random.default_rng(T + HI)
    nq, B = 2, 2
    iq, iw, ik = int_inputs(rng, nq, B, T, HI, DI, r, 3)
    cq, ck = e4m3_codes_of(iq), e4m3_codes_of(ik)
    sq = np.ones((nq, HI), dtype=np.float32)
    sk = np.ones((B, T), dtype=np.float32)
    nvis = np.array([T, max(0, T - 5)])
    p8, t8 = indexer_fp8.index_full(cq, sq, iw, ck, sk, 1, nvis)
    pi, ti = indexer.index_full(iq.astype(np.int8), iw, ik.astype(np.int8), 1, nvis)
    assert np.array_equal(p8, pi) and np.array_equal(t8, ti)
    s8 = indexer_fp8.token_scores(cq[0], sq[0], iw[0], ck[0], sk[0])
    si = indexer.token_scores(iq[0], iw[0], ik[0])
    assert np.array_equal(s8, si)
    r8 = indexer_fp8.index_reindex(cq, sq, iw, ck, sk, 1, pi, nvis)
    ri = indexer.index_reindex(iq.astype(np.int8), iw, ik.astype(np.int8), 1, pi, nvis)
    assert np.array_equal(r8, ri)


def test_power_of_two_scales_closed_form():
    rng = np.random.default_rng(3)
    T, HI, DI = 3000, 4, 32
    iq, iw, ik = int_inputs(rng, 1, 1, T, HI, DI, 8, 5)
    e = rng.integers(-6, 7, size=T)
    f = rng.integers(-6, 7, size=HI)
    sk = np.ldexp(1.0, e).astype(np.float32)
    sq = np.ldexp(1.0, f).astype(np.float32)
    s8 = indexer_fp8.token_scores(e4m3_codes_of(iq[0]), sq, iw[0], e4m3_codes_of(ik[0]), sk)
    # s(t) = 2^e_t * sum_h (w_h 2^f_h) relu(q_h . k_t): every step exact in FP64
    si = indexer.token_scores(iq[0], iw[0].astype(np.float64) * np.ldexp(1.0, f), ik[0])
    assert np.array_equal(s8, np.ldexp(si, e))
    assert np.any(s8 > 0) and np.any(s8 == 0)


def test_relu_sign_identities():
    rng = np.random.default_rng(4)
    T, HI, DI = 500, 8, 128
    cq = finite_codes(rng, (HI, DI))
    ck = finite_codes(rng, (T, DI))
    sq = (rng.random(HI) + 0.5).astype(np.float32)
    sk = (rng.random(T) + 0.5).astype(np.float32)
    iw = (rng.random(HI) * 2 - 0.5).astype(np.float32)
    s_pos = indexer_fp8.token_scores(cq, sq, iw, ck, sk)
    s_neg = indexer_fp8.token_scores(cq, sq, iw, ck ^ 0x80, sk)      # every key negated
    qk = (e4m3_decode(ck) * sk[:, None].astype(np.float64)) @ (e4m3_decode(cq) * sq[:, None].astype(np.float64)).T
    w = iw.astype(np.float64)
    lin = qk @ w
    absf = np.abs(qk) @ w
    scale = np.abs(qk) @ np.abs(w)
    assert np.all(np.abs((s_pos - s_neg) - lin) <= 1e-12 * scale)
    assert np.all(np.abs((s_pos + s_neg) - absf) <= 1e-12 * scale)
    a = indexer_fp8.abs_scores(cq, sq, iw, ck, sk)
    elem = ((np.abs(e4m3_decode(ck)) * sk[:, None].astype(np.float64))
            @ (np.abs(e4m3_decode(cq)) * sq[:, None].astype(np.float64)).T) @ np.abs(w)
    assert np.all(np.abs(a - elem) <= 1e-12 * elem)
    assert np.all(scale <= a * (1 + 1e-12)) and np.all(np.abs(s_pos) <= a * (1 + 1e-12))


def test_abs_scores_equal_scores_when_all_terms_positive():
    rng = np.random.default_rng(5)
    cq = rng.integers(0x08, 0x70, size=(4, 16)).astype(np.uint8)     # positive normal values
    ck = rng.integers(0x08, 0x70, size=(50, 16)).astype(np.uint8)
    sq = (rng.random(4) + 0.5).astype(np.float32)
    sk = (rng.random(50) + 0.5).astype(np.float32)
    iw = (rng.random(4) + 0.1).astype(np.float32)
    s = indexer_fp8.token_scores(cq, sq, iw, ck, sk)
    a = indexer_fp8.abs_scores(cq, sq, iw, ck, sk)
    assert np.allclose(s, a, rtol=1e-14, atol=0)


def _exact_scores(cq, sq, iw, ck, sk):
    qv = [[Fraction(float(v)) for v in row] for row in e4m3_decode(cq)]
    kv = [[Fraction(float(v)) for v in row] for row in e4m3_decode(ck)]
    out = []
    for t in range(len(kv)):
        s = Fraction(0)
        for h in range(len(qv)):
            d = sum(a * b for a, b in zip(qv[h], kv[t])) * Fraction(float(sq[h])) * Fraction(float(sk[t]))
            s += Fraction(float(iw[h])) * max(Fraction(0), d)
        out.append(s)
    return out


@pytest.mark.parametrize("T", [7, 600, 20000])
def test_brute_force_exact_rationals(T):
    rng = np.random.default_rng(T)
    HI, DI = 2, 4
    cq = finite_codes(rng, (1, HI, DI))
    ck = finite_codes(rng, (1, T, DI))
    sq = (rng.random((1, HI)) + 0.5).astype(np.float32)
    sk = (rng.random((1, T)) + 0.5).astype(np.float32)
    iw = (rng.random((1, HI)) * 1.5 - 0.25).astype(np.float32)
    s = _exact_scores(cq[0], sq[0], iw[0], ck[0], sk[0])
    nb = (T + 7) // 8
    bmax = [max(s[8 * b: min(8 * b + 8, T)]) for b in range(nb)]
    blocks = sorted(sorted(range(nb), key=lambda b: (-bmax[b], b))[:2048])
    cand = [8 * b + r for b in blocks for r in range(8) if 8 * b + r < T]
    top = sorted(sorted(cand, key=lambda t: (-s[t], t))[:512])
    pool, topk = indexer_fp8.index_full(cq, sq, iw, ck, sk, 1)
    assert list(pool[0][pool[0] >= 0]) == blocks
    assert list(topk[0][topk[0] >= 0]) == top
    so = indexer_fp8.token_scores(cq[0], sq[0], iw[0], ck[0], sk[0])
    ex = np.array([float(v) for v in s])
    assert np.all(np.abs(so - ex) <= 1e-15 * np.abs(ex) + 1e-300)


@pytest.mark.parametrize("seed", [0, 1])
def test_pool_topk_equals_global_and_scale_invariance(seed):
    rng = np.random.default_rng(seed)
    T, HI, DI = 40000, 4, 16
    cq = finite_codes(rng, (1, HI, DI))
    ck = finite_codes(rng, (1, T, DI))
    sq = (rng.random((1, HI)) + 0.5).astype(np.float32)
    sk = (rng.random((1, T)) + 0.5).astype(np.float32)
    iw = (rng.random((1, HI)) * 1.25 - 0.25).astype(np.float32)
    pool, topk = indexer_fp8.index_full(cq, sq, iw, ck, sk, 1)
    g = indexer_fp8.global_topk(cq[0], sq[0], iw[0], ck[0], sk[0], T)
    assert np.array_equal(topk[0][topk[0] >= 0], g)
    pool2, topk2 = indexer_fp8.index_full(cq, sq, iw, ck, (sk * 2).astype(np.float32), 1)
    assert np.array_equal(pool, pool2) and np.array_equal(topk, topk2)
    assert (pool[0] >= 0).sum() == 2048 and (topk[0] >= 0).sum() == 512
