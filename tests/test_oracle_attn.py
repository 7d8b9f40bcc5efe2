"""Pins of the oracle's sparse + sliding-window attention (CPU only).

Closed forms (Q = 0 gives the mean of the entries; a dominant logit gives
that entry), torch's float64 scaled_dot_product_attention on the gathered
entries (library routine), a pure-Python brute force on a tiny case, Top-K
order invariance, the causal window for several queries per sequence and the
empty / partial-window cases."""
import math

import numpy as np
import torch

from oracle import attention, formats, quant


def _setup(rng, B=2, T=300, d=64, H=4, W=16, Qn=1, k=40):
    x = rng.standard_normal((B * T, d)).astype(np.float32)
    codes, scales = quant.quantize_rows(x)
    q = rng.standard_normal((B * Qn, H, d))
    swa = rng.standard_normal((B, W - 1 + Qn, d))
    topk = np.full((B * Qn, k), -1, dtype=np.int32)
    for qi in range(B * Qn):
        n = rng.integers(1, k + 1)
        topk[qi, :n] = np.sort(rng.choice(T, size=n, replace=False))
    return codes, scales, q, swa, topk


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(0)
    B, T, d, H, W, Qn = 2, 300, 64, 4, 16, 3
    codes, scales, q, swa, topk = _setup(rng, B, T, d, H, W, Qn)
    out = attention.sparse_attn(q, codes, scales, topk, swa, Qn, T, window=W)
    for qi in range(B * Qn):
        b, j = divmod(qi, Qn)
        pos = topk[qi][topk[qi] >= 0]
        kv = np.concatenate([formats.dequant_rows(codes[b * T + pos], scales[b * T + pos], d),
                             swa[b, j:j + W]])
        kt = torch.from_numpy(kv)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[qi])[None, :, None, :].transpose(1, 2).transpose(1, 2).reshape(1, H, 1, d),
            kt.expand(1, H, -1, -1), kt.expand(1, H, -1, -1))
        np.testing.assert_allclose(out[qi], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean():
    rng = np.random.default_rng(1)
    codes, scales, q, swa, topk = _setup(rng)
    q[:] = 0.0
    out = attention.sparse_attn(q, codes, scales, topk, swa, 1, 300, window=16)
    for qi in range(2):
        keys = attention.query_entries(qi, 1, 300, topk[qi], codes, scales, swa, 16)
        np.testing.assert_allclose(out[qi], np.broadcast_to(keys.mean(axis=0), out[qi].shape),
                                   rtol=1e-13, atol=1e-13)


def test_dominant_logit_selects_entry():
    rng = np.random.default_rng(2)
    codes, scales, q, swa, topk = _setup(rng, B=1, W=16)
    target = swa[0, 5] / np.linalg.norm(swa[0, 5])
    q[0] = 400.0 * target          # logit gap >> 1 toward SWA row 5
    out = attention.sparse_attn(q, codes, scales, topk, swa, 1, 300, window=16)
    np.testing.assert_allclose(out[0], np.broadcast_to(swa[0, 5], out[0].shape), atol=1e-6)


def test_pure_python_brute_force_tiny():
    rng = np.random.default_rng(3)
    codes, scales, q, swa, topk = _setup(rng, B=1, T=20, d=16, H=2, W=4, k=5)
    out = attention.sparse_attn(q, codes, scales, topk, swa, 1, 20, window=4)
    pos = [int(t) for t in topk[0] if t >= 0]
    rows = [[formats.e2m1_value((int(codes[p, c // 2]) >> (4 * (c % 2))) & 0xF)
             * formats.e4m3_value(int(scales[p, c // 16])) for c in range(16)] for p in pos]
    rows += [list(swa[0, r]) for r in range(4)]
    for h in range(2):
        logits = [sum(q[0, h, c] * row[c] for c in range(16)) / math.sqrt(16) for row in rows]
        m = max(logits)
        p = [math.exp(v - m) for v in logits]
        for c in range(16):
            ref = math.fsum(pi * row[c] for pi, row in zip(p, rows)) / math.fsum(p)
            assert abs(out[0, h, c] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_topk_order_invariance_and_empty_slots():
    rng = np.random.default_rng(4)
    codes, scales, q, swa, topk = _setup(rng)
    a = attention.sparse_attn(q, codes, scales, topk, swa, 1, 300, window=16)
    perm = topk.copy()
    for qi in range(2):
        rng.shuffle(perm[qi])                       # -1 slots move around too
    b = attention.sparse_attn(q, codes, scales, perm, swa, 1, 300, window=16)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_empty_topk_is_dense_window_attention():
    rng = np.random.default_rng(5)
    codes, scales, q, swa, topk = _setup(rng)
    topk[:] = -1
    out = attention.sparse_attn(q, codes, scales, topk, swa, 1, 300, window=16)
    for qi in range(2):
        k = torch.from_numpy(swa[qi])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[qi])[None, :, None, :].reshape(1, 4, 1, 64), k.expand(1, 4, -1, -1),
            k.expand(1, 4, -1, -1))
        np.testing.assert_allclose(out[qi], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_causal_window_and_partial_window():
    rng = np.random.default_rng(6)
    B, T, d, H, W, Qn = 1, 50, 32, 2, 8, 4
    codes, scales, q, swa, topk = _setup(rng, B, T, d, H, W, Qn, k=3)
    topk[:] = -1
    out = attention.sparse_attn(q, codes, scales, topk, swa, Qn, T, window=W)
    for j in range(Qn):               # query j sees rows j .. j+W-1
        ref = attention.attend(q[j], swa[0, j:j + W], 1 / math.sqrt(d))
        np.testing.assert_allclose(out[j], ref, rtol=1e-13, atol=1e-13)
    # only the last 5 rows are valid: query j sees rows max(j, 6) .. j+W-1
    swa_len = np.array([5])
    out = attention.sparse_attn(q, codes, scales, topk, swa, Qn, T, window=W, swa_len=swa_len)
    for j in range(Qn):
        lo = max(j, W - 1 + Qn - 5)
        ref = attention.attend(q[j], swa[0, lo:j + W], 1 / math.sqrt(d))
        np.testing.assert_allclose(out[j], ref, rtol=1e-13, atol=1e-13)
    # nothing valid at all -> zeros
    out = attention.sparse_attn(q, codes, scales, topk, swa, Qn, T, window=W, swa_len=np.array([0]))
    assert np.all(out == 0.0)
