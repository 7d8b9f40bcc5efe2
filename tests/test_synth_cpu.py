"""The seeded input recipes (CPU only): shapes, value ranges and determinism
of what fp4_kv_cache_e4m3_amd.synth draws, as the workloads document them."""
import numpy as np
import torch

from fp4_kv_cache_e4m3_amd import synth


def small(**kw):
    return synth.Small(batch=3, kv_len=5000, dim=128, heads=8, idx_heads=4, idx_dim=64).workload().replace(**kw)


def e4m3(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_indexer_inputs():
    w = small(idx_fp8=True)
    ik = synth.index_k_all(w)
    iq = synth.index_q(w)
    assert ik.dtype == np.uint8 and ik.shape == (w.batch, w.kv_len, w.idx_dim)
    assert iq.dtype == np.uint8 and iq.shape == (w.nq, w.idx_heads, w.idx_dim)
    for c in (ik, iq):
        mag = np.abs(e4m3(c))
        assert mag.min() == 0.25 and mag.max() == 15.0                  # the 48 magnitudes 0.25 .. 15
        assert len(np.unique(c)) == 96                                   # and both signs
        assert 0.45 < np.mean(c >= 0x80) < 0.55
    sk, sq = synth.index_k_scale_all(w), synth.index_q_scale(w)
    assert sk.shape == (w.batch, w.kv_len) and sq.shape == (w.nq, w.idx_heads)
    for s in (sk, sq):
        assert s.dtype == np.float32 and s.min() >= 1 / 32 and s.max() < 1 / 16
    iw = synth.index_w(w)
    assert iw.dtype == np.float32 and iw.min() >= -0.25 and iw.max() < 1.0 and iw.min() < 0
    np.testing.assert_array_equal(synth.index_k_all(w), ik)              # seeded: the same draw again
    np.testing.assert_array_equal(synth.index_k_rows(w, 1, 4090, 20), ik[1, 4090:4110])   # any chunk on its own


def test_integer_indexer_inputs():
    w = small()
    ik, iq, iw = synth.index_k_all(w), synth.index_q(w), synth.index_w(w)
    assert ik.dtype == np.int8 and iq.dtype == np.int8
    assert ik.min() == -w.idx_range and ik.max() == w.idx_range
    assert np.all(iw == np.round(iw)) and iw.min() >= 1 and iw.max() <= w.w_max


def test_paged_layout_and_ring_starts():
    w = small(page_size=256, swa_ring=True)
    per_seq, n_phys = synth.page_count(w)
    assert per_seq == (w.kv_len + 255) // 256 and n_phys == (w.batch + 1) * per_seq
    bt = synth.block_table(w)
    assert bt.shape == (w.batch, per_seq) and bt.dtype == np.int32
    assert len(np.unique(bt)) == bt.size and bt.min() >= 0 and bt.max() < n_phys   # distinct pages
    st = synth.swa_ring_start(w, 2)
    assert st.shape == (w.batch,) and st.min() >= 0 and st.max() < w.swa_rows


def test_new_window_rows():
    w = small(swa8=True)
    nb = synth.new_swa_rows(w, 1)
    assert nb.shape == (w.nq, w.dim) and nb.dtype == np.uint16
    assert not np.array_equal(nb, synth.new_swa_rows(w, 2))               # per layer
