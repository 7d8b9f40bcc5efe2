"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (no launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import fp4_kv_cache_e4m3_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libcsa2.so not built (run __graft_entry__.build())")
    return m.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    import fp4_kv_cache_e4m3_amd as m
    names = header_functions()
    assert names == sorted(m.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_declares_every_signature(lib):
    """Every exported function that takes arguments has ctypes argtypes: without
    them ctypes passes a Python int as a 32-bit C int, which truncates device
    pointers."""
    import fp4_kv_cache_e4m3_amd as m
    for n in m.EXPORTS:
        if n == "csa2_version":
            continue
        assert getattr(lib, n).argtypes is not None, n


def test_status_strings(lib):
    import fp4_kv_cache_e4m3_amd as m
    for s in range(6):
        assert m.status_string(s).startswith("CSA2_")
    assert lib.csa2_version() >> 16 == 1


def test_quantize_rejects(lib):
    f = lib.csa2_quantize_kv
    assert f(None, 512, 4, 33, None, 256, None, 32, None) == 2            # dim % 32
    assert f(None, 512, 4, 512, None, 256, None, 32, None) == 1           # NULL x
    assert f(16, 512, 4, 512, 16, 100, 16, 32, None) == 2                 # codes stride < d/2
    assert f(8, 512, 4, 512, 16, 256, 16, 32, None) == 3                  # x misaligned
    assert f(None, 512, 0, 512, None, 256, None, 32, None) == 0           # empty: no-op


def test_quantize_swa_fp8_rejects(lib):
    f = lib.csa2_quantize_swa_fp8
    assert f(16, 512, 4, 12, 16, 512, 16, 1, None) == 2                    # dim % 8
    assert f(16, 1024, 4, 1024, 16, 1024, 16, 1, None) == 2                # dim > 512
    assert f(None, 512, 4, 512, 16, 512, 16, 1, None) == 1                 # NULL x
    assert f(16, 512, 4, 512, 16, 256, 16, 1, None) == 2                   # out stride < dim
    assert f(16, 512, 4, 512, 16, 512, 16, 0, None) == 2                   # scale stride < 1
    assert f(8, 512, 4, 512, 16, 512, 16, 1, None) == 3                    # x misaligned
    assert f(16, 512, 4, 512, 16, 512, 18, 1, None) == 3                   # scales misaligned
    assert f(None, 512, 0, 512, None, 512, None, 1, None) == 0             # empty: no-op


def test_index_rejects(lib):
    import fp4_kv_cache_e4m3_amd as m
    a = m.IndexArgs(1, 1, 100, 3, 64, 16, 16, 16, None)                    # 3 heads
    assert lib.csa2_index_full(ctypes.byref(a), None, 16, None, 0, None) == 2
    assert lib.csa2_index_workspace_size(ctypes.byref(a)) == 0
    a = m.IndexArgs(1, 262141, 100, 16, 64, 16, 16, 16, None)              # Qn*H_I > 64*65535
    assert lib.csa2_index_full(ctypes.byref(a), None, 16, None, 0, None) == 2
    a = m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None)
    ws = lib.csa2_index_workspace_size(ctypes.byref(a))
    assert ws > 0 and ws % 256 == 0
    assert lib.csa2_index_full(ctypes.byref(a), None, 16, 256, ws - 1, None) == 4
    assert lib.csa2_index_full(ctypes.byref(a), None, 16, None, ws, None) == 4
    assert lib.csa2_index_full(ctypes.byref(a), None, None, 256, ws, None) == 1
    a = m.IndexArgs(1, 1, 100, 8, 64, 17, 16, 16, None)                    # iq misaligned
    assert lib.csa2_index_full(ctypes.byref(a), None, 16, 256, ws, None) == 3
    assert lib.csa2_index_reindex(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None)),
                                  None, 16, 256, ws, None) == 1            # no pool
    a = m.IndexArgs(1, 1, (1 << 20) + 1, 8, 64, 16, 16, 16, None)          # T too long
    assert lib.csa2_index_workspace_size(ctypes.byref(a)) == 0
    # from 2^19 positions on, the scan keeps only block maxima: the workspace
    # shrinks from 4.5 B per query and position to 0.5 B (plus the pool, its
    # blocks' keys and a key floor per query)
    short = lib.csa2_index_workspace_size(ctypes.byref(m.IndexArgs(1, 2, (1 << 19) - 16, 8, 64, 16, 16, 16, None)))
    long_ = lib.csa2_index_workspace_size(ctypes.byref(m.IndexArgs(1, 2, 1 << 19, 8, 64, 16, 16, 16, None)))
    up = lambda x, m: (x + m - 1) // m * m
    assert short == up(2 * (((1 << 19) - 16) + up(((1 << 19) - 16) // 8, 16)) * 4, 256)
    assert long_ == up(2 * (1 << 16) * 4 + 2 * 2048 * 4 + 2 * 2048 * 4 + 2 * 4, 256)


def test_check_index_rejects(lib):
    import fp4_kv_cache_e4m3_amd as m
    a = m.IndexArgs(1, 2, 100, 8, 64, 16, 16, 16, None)
    f = lib.csa2_check_index
    assert f(ctypes.byref(a), 16, 16, 3, 16, None) == 2          # mode
    assert f(ctypes.byref(a), 16, 16, 0, None, None) == 1        # no counter
    assert f(ctypes.byref(a), 16, None, 0, 16, None) == 1        # no Top-K in mode 0
    assert f(ctypes.byref(a), None, 16, 1, 16, None) == 1        # no pool in mode 1
    assert f(ctypes.byref(a), None, None, 2, 16, None) == 1      # no pool in mode 2
    assert f(ctypes.byref(a), 16, 16, 0, 18, None) == 3          # misaligned counter
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 3, 64, 16, 16, 16, None)), 16, 16, 0, 16, None) == 2
    assert f(ctypes.byref(m.IndexArgs(0, 1, 100, 8, 64, 16, 16, 16, None)), None, None, 0, None, None) == 0
    assert lib.csa2_status_string(7).startswith(b"CSA2_ERR_DEBUG")


def test_quantize_bf16_rejects(lib):
    """bf16 rows: 16-byte aligned start and a row stride of a multiple of 8
    elements; the other checks as for fp32 rows."""
    f = lib.csa2_quantize_kv_bf16
    assert f(16, 64, 2, 48, 16, 32, 16, 4, None) == 2             # dim % 32
    assert f(None, 64, 2, 64, 16, 32, 16, 4, None) == 1           # no input
    assert f(16, 60, 2, 64, 16, 32, 16, 4, None) == 2             # stride < dim
    assert f(24, 64, 2, 64, 16, 32, 16, 4, None) == 3             # misaligned rows
    assert f(16, 68, 2, 64, 16, 32, 16, 4, None) == 3             # stride not a multiple of 8
    assert f(16, 64, 0, 64, None, 0, None, 0, None) == 0          # no rows: no-op


def test_read_rate_rejects(lib):
    """The read-rate probe: NULL buffer or sink, a misaligned buffer or sink, or
    a size not a multiple of 16 is refused before any launch; 0 bytes is a
    no-op."""
    f = lib.csa2_read_rate
    assert f(None, 64, 16, None) == 1
    assert f(16, 64, None, None) == 1
    assert f(24, 64, 16, None) == 3
    assert f(16, 60, 16, None) == 3
    assert f(16, 64, 18, None) == 3
    assert f(None, 0, None, None) == 0


def test_index_fp8_rejects(lib):
    """FP8 indexer arguments: the flag must be 0 or 1 and both scale arrays
    present and 4-byte aligned; int8 arguments ignore the scale pointers."""
    import fp4_kv_cache_e4m3_amd as m
    a = m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None)
    ws = lib.csa2_index_workspace_size(ctypes.byref(a))
    f = lib.csa2_index_full
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 2, 16, 16)), None, 16, 256, ws, None) == 2
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, None, 16)), None, 16, 256, ws, None) == 1
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, 16, None)), None, 16, 256, ws, None) == 1
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, 18, 16)), None, 16, 256, ws, None) == 3
    assert f(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, 16, 18)), None, 16, 256, ws, None) == 3
    assert lib.csa2_index_reindex(ctypes.byref(m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, 16, None)),
                                  16, 16, 256, ws, None) == 1
    b = m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None, 1, 16, 16)
    assert lib.csa2_index_workspace_size(ctypes.byref(b)) == ws
    # 32 score rows per scan workgroup with fp8: Qn * H_I <= 32 * 65535
    assert lib.csa2_index_workspace_size(ctypes.byref(m.IndexArgs(1, 131070, 100, 16, 64, 16, 16, 16, None, 1, 16, 16))) > 0
    assert lib.csa2_index_workspace_size(ctypes.byref(m.IndexArgs(1, 131071, 100, 16, 64, 16, 16, 16, None, 1, 16, 16))) == 0
    assert lib.csa2_index_workspace_size(ctypes.byref(m.IndexArgs(1, 131071, 100, 16, 64, 16, 16, 16, None))) > 0


def test_index_append_rejects(lib):
    """The fused index + new-row quantisation calls validate both parts
    before launching anything."""
    import fp4_kv_cache_e4m3_amd as m
    a = m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None)
    ws = lib.csa2_index_workspace_size(ctypes.byref(a))
    for f in (lib.csa2_index_full_append, lib.csa2_index_select_append):
        assert f(ctypes.byref(a), None, 16, 256, ws, 16, 512, 4, 33, 16, 256, 16, 32, None) == 2    # dim % 32
        assert f(ctypes.byref(a), None, 16, 256, ws, None, 512, 4, 512, 16, 256, 16, 32, None) == 1  # NULL x
        assert f(ctypes.byref(a), None, 16, 256, ws, 8, 512, 4, 512, 16, 256, 16, 32, None) == 3     # x misaligned
        assert f(ctypes.byref(a), None, 16, 256, ws - 1, 16, 512, 4, 512, 16, 256, 16, 32, None) == 4  # workspace
        bad = m.IndexArgs(1, 1, 100, 3, 64, 16, 16, 16, None)                                       # 3 heads
        assert f(ctypes.byref(bad), None, 16, 256, ws, 16, 512, 4, 512, 16, 256, 16, 32, None) == 2


def test_paged_rejects(lib):
    """Paged-cache and window-ring arguments are validated before any launch:
    page size a power of two in 1 .. 65536, enough pages for T, the cache
    within 2^24 rows and 4 GiB, 4-byte alignment; no compute runs (no GPU)."""
    import fp4_kv_cache_e4m3_amd as m

    def args(**kw):
        base = dict(batch=2, q_per_seq=1, kv_len=64, heads=16, dim=512, q=256, codes=256,
                    codes_stride=256, scales=256, scales_stride=32, topk=256, topk_k=512, swa=256,
                    window=128, swa_len=None, sm_scale=0.0, out=256, block_table=256, max_pages=4,
                    page_size=16, cache_rows=1024)
        base.update(kw)
        return m.AttnArgs(**base)

    sa = lib.csa2_attn_workspace_size
    assert sa(ctypes.byref(args())) > 0
    assert sa(ctypes.byref(args(page_size=24))) == 0            # not a power of two
    assert sa(ctypes.byref(args(page_size=0))) == 0
    assert sa(ctypes.byref(args(page_size=1 << 17))) == 0
    assert sa(ctypes.byref(args(max_pages=3))) == 0              # 3 x 16 < T = 64
    assert sa(ctypes.byref(args(cache_rows=1 << 24))) == 0
    assert sa(ctypes.byref(args(cache_rows=-1))) == 0
    assert lib.csa2_sparse_attn(ctypes.byref(args(block_table=258)), None, 0, None) == 3
    assert lib.csa2_sparse_attn(ctypes.byref(args(swa_start=258)), None, 0, None) == 3
    q = lib.csa2_quantize_kv_paged
    #        x    xs   rows dim  seq  pos  bt   B  maxp ps  codes cs   scales ss rows_c stream
    assert q(16, 512, 4, 512, 16, 16, 16, 2, 4, 24, 16, 256, 16, 32, 64, None) == 2     # page size
    assert q(16, 512, 4, 512, 16, 16, 16, 0, 4, 16, 16, 256, 16, 32, 64, None) == 2     # batch
    assert q(16, 512, 4, 512, None, 16, 16, 2, 4, 16, 16, 256, 16, 32, 64, None) == 1   # no row_seq
    assert q(16, 512, 4, 512, 16, 16, None, 2, 4, 16, 16, 256, 16, 32, 64, None) == 1   # no table
    assert q(16, 512, 4, 512, 18, 16, 16, 2, 4, 16, 16, 256, 16, 32, 64, None) == 3     # misaligned
    assert q(16, 512, 4, 33, 16, 16, 16, 2, 4, 16, 16, 256, 16, 32, 64, None) == 2      # dim % 32
    assert q(None, 512, 0, 512, None, None, None, 2, 4, 16, None, 256, None, 32, 64, None) == 0   # empty
    # the fused index + paged new-row calls validate both parts first
    ia = m.IndexArgs(1, 1, 100, 8, 64, 16, 16, 16, None)
    ws = lib.csa2_index_workspace_size(ctypes.byref(ia))
    for f in (lib.csa2_index_full_append_paged, lib.csa2_index_select_append_paged):
        ok = (16, 512, 4, 512, 16, 16, 16, 2, 4, 16, 16, 256, 16, 32, 64)
        assert f(ctypes.byref(ia), None, 16, 256, ws, *ok[:9], 24, *ok[10:], None) == 2           # page size
        assert f(ctypes.byref(ia), None, 16, 256, ws, *ok[:6], None, *ok[7:], None) == 1          # no table
        assert f(ctypes.byref(ia), None, 16, 256, ws - 1, *ok, None) == 4                         # workspace
        bad = m.IndexArgs(1, 1, 100, 3, 64, 16, 16, 16, None)                                      # 3 heads
        assert f(ctypes.byref(bad), None, 16, 256, ws, *ok, None) == 2


def test_attn_rejects(lib):
    import fp4_kv_cache_e4m3_amd as m

    def args(**kw):
        base = dict(batch=2, q_per_seq=1, kv_len=64, heads=16, dim=512, q=256, codes=256,
                    codes_stride=256, scales=256, scales_stride=32, topk=256, topk_k=512, swa=256,
                    window=128, swa_len=None, sm_scale=0.0, out=256)
        base.update(kw)
        return m.AttnArgs(**base)

    sa = lib.csa2_sparse_attn
    assert sa(ctypes.byref(args(dim=256)), None, 0, None) == 2
    assert sa(ctypes.byref(args(topk_k=4096)), None, 0, None) == 2
    assert sa(ctypes.byref(args(q=None)), None, 0, None) == 1
    assert sa(ctypes.byref(args(codes_stride=200)), None, 0, None) == 2
    assert sa(ctypes.byref(args(codes_stride=264)), None, 0, None) == 3
    assert sa(ctypes.byref(args(out=260)), None, 0, None) == 3
    a = args()
    need = lib.csa2_attn_workspace_size(ctypes.byref(a))
    assert need > 0                                   # 2 queries x 4 head groups -> split
    assert sa(ctypes.byref(a), None, 0, None) == 4
    assert sa(ctypes.byref(a), 256, need - 1, None) == 4
    # the caller's work split: waves 4 or 8, splits >= 0 (0 = the library's choice)
    assert sa(ctypes.byref(args(waves=5)), None, 0, None) == 2
    assert sa(ctypes.byref(args(splits=-1)), None, 0, None) == 2
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(waves=8, splits=1))) == 0
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(waves=4, splits=3))) > 0
    # kernel: 0 the library's choice, 1 head groups, 2 one workgroup per query
    # (dim 512, bf16 window, no explicit waves / splits; never a workspace)
    assert sa(ctypes.byref(args(kernel=3)), None, 0, None) == 2
    assert sa(ctypes.byref(args(kernel=-1)), None, 0, None) == 2
    assert sa(ctypes.byref(args(kernel=2, dim=128, codes_stride=64, scales_stride=8)), None, 0, None) == 2
    assert sa(ctypes.byref(args(kernel=2, waves=4)), None, 0, None) == 2
    assert sa(ctypes.byref(args(kernel=2, splits=2)), None, 0, None) == 2
    assert sa(ctypes.byref(args(kernel=2, swa_fp8=1, swa_scale=256)), None, 0, None) == 2
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(kernel=2))) == 0
    # the library's choice for a prefill chunk (4,096 queries): no workspace
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(batch=1, q_per_seq=4096))) == 0
    # new 8-bit window rows encoded by the call: 8-bit windows of at least one
    # row, at most 16 query tokens per sequence, 16-byte aligned
    s8 = dict(swa_fp8=1, swa_scale=256)
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(swa_new=256, **s8))) == need     # accepted
    assert sa(ctypes.byref(args(swa_new=256)), None, 0, None) == 2                      # bf16 window
    assert sa(ctypes.byref(args(swa_new=256, window=0, **s8)), None, 0, None) == 2      # no window
    assert sa(ctypes.byref(args(swa_new=256, batch=1, q_per_seq=17, **s8)), None, 0, None) == 2
    assert sa(ctypes.byref(args(swa_new=264, **s8)), None, 0, None) == 3
    # the Top-K as cache rows: written by a paged call, read without a block table
    pg = dict(block_table=256, max_pages=4, page_size=16, cache_rows=1024)
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(topk_rows_out=256, **pg))) == need   # accepted
    assert lib.csa2_attn_workspace_size(ctypes.byref(args(topk_is_rows=1, cache_rows=1024))) == need
    assert sa(ctypes.byref(args(topk_rows_out=256)), None, 0, None) == 2                 # no block table
    assert sa(ctypes.byref(args(topk_rows_out=258, **pg)), None, 0, None) == 3
    assert sa(ctypes.byref(args(topk_rows_out=256, kernel=2, **pg)), None, 0, None) == 2
    assert sa(ctypes.byref(args(topk_is_rows=1, cache_rows=1024, block_table=256, max_pages=4, page_size=16)),
              None, 0, None) == 2
    assert sa(ctypes.byref(args(topk_is_rows=2, cache_rows=1024)), None, 0, None) == 2
    assert sa(ctypes.byref(args(topk_is_rows=1, cache_rows=1 << 24)), None, 0, None) == 2


def test_argument_structs_keep_their_tensors_alive():
    """index_args / attn_args hold raw pointers; the structs also hold the
    tensors, so a caller dropping its own references cannot free memory that
    a later call reads (the caching allocator would hand it out again)."""
    import gc
    import weakref

    import torch

    import fp4_kv_cache_e4m3_amd as m

    iq = torch.zeros((2, 8, 128), dtype=torch.int8)
    iw, ik = torch.ones((2, 8)), torch.zeros((2, 64, 128), dtype=torch.int8)
    refs = [weakref.ref(t) for t in (iq, iw, ik)]
    ia = m.index_args(iq, iw, ik, 1)
    del iq, iw, ik
    gc.collect()
    assert all(r() is not None for r in refs)
    assert ia.q == ia._keep[0].data_ptr()
    del ia
    gc.collect()
    assert all(r() is None for r in refs)

    q = torch.zeros((2, 16, 128), dtype=torch.int16)
    codes, scales = torch.zeros((128, 64), dtype=torch.uint8), torch.zeros((128, 8), dtype=torch.uint8)
    topk, swa = torch.zeros((2, 64), dtype=torch.int32), torch.zeros((2, 127, 128), dtype=torch.int16)
    out = torch.zeros((2, 16, 128))
    ts = (q, codes, scales, topk, swa, out)
    refs = [weakref.ref(t) for t in ts]
    aa = m.attn_args(*ts, 1, 64, 128, waves=4, splits=2)
    del ts, q, codes, scales, topk, swa, out
    gc.collect()
    assert all(r() is not None for r in refs)
    assert (aa.waves, aa.splits) == (4, 2)
    del aa
    gc.collect()
    assert all(r() is None for r in refs)
