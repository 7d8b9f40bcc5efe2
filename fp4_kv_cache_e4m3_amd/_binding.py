"""ctypes binding of libcsa2.so (include/csa2.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI and turns a non-zero status into
``CSA2Error``.  All computation happens in the library's gfx950 kernels.
PyTorch supplies device memory and the stream; nothing here falls back to the
CPU -- if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

TOPK = 512
BLOCK = 8
POOL_BLOCKS = 2048
WINDOW = 128
SCALE_GROUP = 16

EXPORTS = (
    "csa2_status_string", "csa2_version", "csa2_quantize_kv", "csa2_quantize_kv_bf16", "csa2_quantize_kv_paged",
    "csa2_quantize_swa_fp8",
    "csa2_dequantize_kv",
    "csa2_index_workspace_size", "csa2_index_full", "csa2_index_scan", "csa2_index_select",
    "csa2_index_full_append", "csa2_index_select_append", "csa2_index_full_append_paged",
    "csa2_index_select_append_paged", "csa2_index_reindex",
    "csa2_attn_workspace_size", "csa2_sparse_attn", "csa2_index_full_noalloc", "csa2_check_index",
    "csa2_read_rate",
)
READ_RATE_SINK_WORDS = 65536


class CSA2Error(RuntimeError):
    pass


class IndexArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32), ("kv_len", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k", ctypes.c_void_p),
        ("n_visible", ctypes.c_void_p),
        ("fp8", ctypes.c_int32), ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32), ("kv_len", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("codes", ctypes.c_void_p), ("codes_stride", ctypes.c_int64),
        ("scales", ctypes.c_void_p), ("scales_stride", ctypes.c_int64),
        ("topk", ctypes.c_void_p), ("topk_k", ctypes.c_int32),
        ("swa", ctypes.c_void_p), ("window", ctypes.c_int32),
        ("swa_len", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("swa_fp8", ctypes.c_int32), ("swa_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("cache_rows", ctypes.c_int64), ("swa_start", ctypes.c_void_p),
        ("waves", ctypes.c_int32), ("splits", ctypes.c_int32), ("kernel", ctypes.c_int32),
        ("swa_new", ctypes.c_void_p),
        ("topk_rows_out", ctypes.c_void_p), ("topk_is_rows", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcsa2.so once; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CSA2Error(f"{path} is missing: build it with `python -m fp4_kv_cache_e4m3_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.csa2_status_string.restype = ctypes.c_char_p
    lib.csa2_status_string.argtypes = [ctypes.c_int]
    lib.csa2_version.restype = ctypes.c_int
    lib.csa2_quantize_kv.restype = ctypes.c_int
    lib.csa2_quantize_kv.argtypes = [vp, i64, i64, i32, vp, i64, vp, i64, vp]
    lib.csa2_quantize_kv_bf16.restype = ctypes.c_int
    lib.csa2_quantize_kv_bf16.argtypes = [vp, i64, i64, i32, vp, i64, vp, i64, vp]
    lib.csa2_quantize_kv_paged.restype = ctypes.c_int
    lib.csa2_quantize_kv_paged.argtypes = [vp, i64, i64, i32, vp, vp, vp, i32, i32, i32, vp, i64, vp, i64, i64, vp]
    for name in ("csa2_index_full_append_paged", "csa2_index_select_append_paged"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp, sz, vp, i64, i64, i32, vp, vp, vp,
                                       i32, i32, i32, vp, i64, vp, i64, i64, vp]
    lib.csa2_quantize_swa_fp8.restype = ctypes.c_int
    lib.csa2_quantize_swa_fp8.argtypes = [vp, i64, i64, i32, vp, i64, vp, i64, vp]
    lib.csa2_dequantize_kv.restype = ctypes.c_int
    lib.csa2_dequantize_kv.argtypes = [vp, i64, vp, i64, i64, i32, vp, i64, vp]
    lib.csa2_index_workspace_size.restype = sz
    lib.csa2_index_workspace_size.argtypes = [ctypes.POINTER(IndexArgs)]
    lib.csa2_index_full.restype = ctypes.c_int
    lib.csa2_index_full.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp, sz, vp]
    lib.csa2_index_full_noalloc.restype = ctypes.c_int
    lib.csa2_index_full_noalloc.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp]
    lib.csa2_index_scan.restype = ctypes.c_int
    lib.csa2_index_scan.argtypes = [ctypes.POINTER(IndexArgs), vp, sz, vp]
    lib.csa2_index_select.restype = ctypes.c_int
    lib.csa2_index_select.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp, sz, vp]
    for name in ("csa2_index_full_append", "csa2_index_select_append"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp, sz, vp, i64, i64, i32, vp, i64, vp, i64, vp]
    lib.csa2_index_reindex.restype = ctypes.c_int
    lib.csa2_index_reindex.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, vp, sz, vp]
    lib.csa2_attn_workspace_size.restype = sz
    lib.csa2_attn_workspace_size.argtypes = [ctypes.POINTER(AttnArgs)]
    lib.csa2_sparse_attn.restype = ctypes.c_int
    lib.csa2_sparse_attn.argtypes = [ctypes.POINTER(AttnArgs), vp, sz, vp]
    lib.csa2_check_index.restype = ctypes.c_int
    lib.csa2_read_rate.restype = ctypes.c_int
    lib.csa2_read_rate.argtypes = [vp, sz, vp, vp]
    lib.csa2_check_index.argtypes = [ctypes.POINTER(IndexArgs), vp, vp, i32, vp, vp]
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int) -> None:
    if status != 0:
        raise CSA2Error(load().csa2_status_string(status).decode())


def status_string(status: int) -> str:
    return load().csa2_status_string(status).decode()


# ------------------------------------------------------------------ quantise
def quantize_kv(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """FP4-quantise fp32 or bf16 rows x [rows, d] into codes [rows, >=d/2] / scales
    [rows, >=d/16] (row strides taken from the tensors, so views into a larger
    cache work); bf16 rows go to csa2_quantize_kv_bf16."""
    rows, dim = x.shape
    fn = load().csa2_quantize_kv_bf16 if x.dtype == torch.bfloat16 else load().csa2_quantize_kv
    _check(fn(_ptr(x), x.stride(0), rows, dim, _ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0),
              _stream(stream)))


def quantize_kv_paged(x: torch.Tensor, row_seq: torch.Tensor, row_pos: torch.Tensor, block_table: torch.Tensor,
                      page_size: int, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """FP4-quantise fp32 rows x [rows, d] into a paged cache: row r to position
    row_pos[r] of sequence row_seq[r] through block_table int32 [B, max_pages];
    codes [cache_rows, >=d/2] / scales [cache_rows, >=d/16]."""
    rows, dim = x.shape
    B, max_pages = block_table.shape
    _check(load().csa2_quantize_kv_paged(_ptr(x), x.stride(0), rows, dim, _ptr(row_seq), _ptr(row_pos),
                                         _ptr(block_table), B, max_pages, page_size, _ptr(codes), codes.stride(0),
                                         _ptr(scales), scales.stride(0), codes.shape[0], _stream(stream)))


def quantize_swa_fp8(x: torch.Tensor, out: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """8-bit window rows: bf16 bits x [rows, d] (int16/uint16 storage) -> E4M3
    codes out [rows, >=d] (uint8) and power-of-two row scales [rows] (fp32,
    any row stride)."""
    rows, dim = x.shape
    _check(load().csa2_quantize_swa_fp8(_ptr(x), x.stride(0), rows, dim, _ptr(out), out.stride(0), _ptr(scales),
                                        scales.stride(0), _stream(stream)))


def dequantize_kv(codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    rows, dim = out.shape
    _check(load().csa2_dequantize_kv(_ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0),
                                     rows, dim, _ptr(out), out.stride(0), _stream(stream)))


# ------------------------------------------------------------------ indexer
def index_args(iq, iw, ik, q_per_seq: int, n_visible=None, q_scale=None, k_scale=None) -> IndexArgs:
    """iq [nq, H_I, D_I], iw fp32 [nq, H_I], ik [B, T, D_I]: int8, or E4M3
    codes (uint8) with q_scale fp32 [nq, H_I] and k_scale fp32 [B, T].
    The struct holds raw device pointers; it also keeps references to the
    tensors they point into, so they live at least as long as the struct."""
    nq, heads, dim = iq.shape
    B, T = ik.shape[0], ik.shape[1]
    fp8 = 1 if (q_scale is not None or k_scale is not None) else 0
    args = IndexArgs(B, q_per_seq, T, heads, dim, _ptr(iq), _ptr(iw), _ptr(ik), _ptr(n_visible),
                     fp8, _ptr(q_scale), _ptr(k_scale))
    args._keep = (iq, iw, ik, n_visible, q_scale, k_scale)   # the tensors its pointers name
    return args


def index_workspace_size(args: IndexArgs) -> int:
    return int(load().csa2_index_workspace_size(ctypes.byref(args)))


def index_full(args: IndexArgs, pool, topk, ws, stream=None) -> None:
    _check(load().csa2_index_full(ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws),
                                  ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def index_full_noalloc(args: IndexArgs, pool, topk, stream=None) -> None:
    """index_full on the library's fixed per-GPU scratch (no workspace, no
    allocation; calls on one GPU must not overlap)."""
    _check(load().csa2_index_full_noalloc(ctypes.byref(args), _ptr(pool), _ptr(topk), _stream(stream)))


def index_scan(args: IndexArgs, ws, stream=None) -> None:
    _check(load().csa2_index_scan(ctypes.byref(args), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def index_select(args: IndexArgs, pool, topk, ws, stream=None) -> None:
    _check(load().csa2_index_select(ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def _append_args(x, codes, scales):
    rows, dim = x.shape
    return (_ptr(x), x.stride(0), rows, dim, _ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0))


def index_full_append(args: IndexArgs, pool, topk, ws, x, codes, scales, stream=None) -> None:
    """index_full plus quantize_kv(x, codes, scales) of the step's new rows."""
    _check(load().csa2_index_full_append(ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws),
                                         ws.numel() * ws.element_size() if ws is not None else 0,
                                         *_append_args(x, codes, scales), _stream(stream)))


def _paged_append_args(x, row_seq, row_pos, block_table, page_size, codes, scales):
    B, max_pages = block_table.shape
    return (_ptr(x), x.stride(0), x.shape[0], x.shape[1], _ptr(row_seq), _ptr(row_pos), _ptr(block_table), B,
            max_pages, page_size, _ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0), codes.shape[0])


def index_full_append_paged(args: IndexArgs, pool, topk, ws, x, row_seq, row_pos, block_table, page_size: int,
                            codes, scales, stream=None) -> None:
    """index_full plus quantize_kv_paged of the step's new rows."""
    _check(load().csa2_index_full_append_paged(
        ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
        *_paged_append_args(x, row_seq, row_pos, block_table, page_size, codes, scales), _stream(stream)))


def index_select_append_paged(args: IndexArgs, pool, topk, ws, x, row_seq, row_pos, block_table, page_size: int,
                              codes, scales, stream=None) -> None:
    """index_select plus quantize_kv_paged of the step's new rows."""
    _check(load().csa2_index_select_append_paged(
        ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
        *_paged_append_args(x, row_seq, row_pos, block_table, page_size, codes, scales), _stream(stream)))


def index_select_append(args: IndexArgs, pool, topk, ws, x, codes, scales, stream=None) -> None:
    """index_select plus quantize_kv(x, codes, scales) of the step's new rows."""
    _check(load().csa2_index_select_append(ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws),
                                           ws.numel() * ws.element_size() if ws is not None else 0,
                                           *_append_args(x, codes, scales), _stream(stream)))


def check_index(args: IndexArgs, pool, topk, mode: int, bad, stream=None) -> None:
    """Device-side check of index rows (mode 0 Full outputs, 1 Reindex
    outputs against the given pool, 2 a Reindex input pool): the number of
    failing rows is added to bad (a device uint32 / int32 scalar tensor)."""
    _check(load().csa2_check_index(ctypes.byref(args), _ptr(pool), _ptr(topk), int(mode), _ptr(bad), _stream(stream)))


def read_rate(buf, sink, stream=None) -> None:
    """Read every byte of buf (a device tensor) once; timing it gives the
    device's achievable HBM read rate.  sink: device int32/uint32 tensor of
    READ_RATE_SINK_WORDS words."""
    _check(load().csa2_read_rate(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def index_reindex(args: IndexArgs, pool, topk, ws, stream=None) -> None:
    _check(load().csa2_index_reindex(ctypes.byref(args), _ptr(pool), _ptr(topk), _ptr(ws),
                                     ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream(stream)))


# ------------------------------------------------------------------ attention
def attn_args(q, codes, scales, topk, swa, out, q_per_seq: int, kv_len: int, window: int = WINDOW,
              swa_len=None, sm_scale: float = 0.0, swa_scale=None, block_table=None, page_size: int = 0,
              swa_start=None, waves: int = 0, splits: int = 0, kernel: int = 0, swa_new=None,
              topk_rows_out=None, topk_is_rows: bool = False) -> AttnArgs:
    """q bf16-as-int16/uint16 [nq, H, d]; codes [B*T, >=d/2]; scales [B*T, >=d/16];
    topk int32 [nq, k]; swa bf16 [B, window-1+Qn, d] -- or, with swa_scale
    (fp32 [B, window-1+Qn]), E4M3 codes uint8 [B, window-1+Qn, d]; out fp32 [nq, H, d].
    Paged cache: block_table int32 [B, max_pages] and page_size, codes / scales
    then hold every physical row.  swa_start int32 [B]: window ring slots.
    waves / splits: the work split (0 = the library's choice); kernel: 0 the
    library's choice, 1 workgroups of 16 heads, 2 one workgroup per query.
    swa_new (8-bit windows only): bf16 [nq, d] new window rows, encoded and
    stored into swa / swa_scale by the call itself.  topk_rows_out (paged):
    int32 [nq, k], the Top-K slots' cache rows written by the call;
    topk_is_rows: topk holds such rows (no block table; codes / scales hold
    every physical row).
    The struct holds raw device pointers; it also keeps references to the
    tensors they point into, so they live at least as long as the struct."""
    nq, heads, dim = q.shape
    paged = block_table is not None
    whole_cache = paged or bool(topk_is_rows)
    args = AttnArgs(nq // q_per_seq, q_per_seq, kv_len, heads, dim, _ptr(q),
                    _ptr(codes), codes.stride(0) if codes is not None else dim // 2,
                    _ptr(scales), scales.stride(0) if scales is not None else dim // 16,
                    _ptr(topk), topk.shape[1] if topk is not None else 0,
                    _ptr(swa), window, _ptr(swa_len), float(sm_scale), _ptr(out),
                    1 if swa_scale is not None else 0, _ptr(swa_scale),
                    _ptr(block_table), block_table.shape[1] if paged else 0, page_size if paged else 0,
                    codes.shape[0] if whole_cache and codes is not None else 0, _ptr(swa_start),
                    int(waves), int(splits), int(kernel), _ptr(swa_new), _ptr(topk_rows_out),
                    1 if topk_is_rows else 0)
    args._keep = (q, codes, scales, topk, swa, out, swa_len, swa_scale, block_table, swa_start, swa_new,
                  topk_rows_out)
    return args


def attn_workspace_size(args: AttnArgs) -> int:
    return int(load().csa2_attn_workspace_size(ctypes.byref(args)))


def sparse_attn(args: AttnArgs, ws=None, stream=None) -> None:
    _check(load().csa2_sparse_attn(ctypes.byref(args), _ptr(ws),
                                   ws.numel() * ws.element_size() if ws is not None else 0,
                                   _stream(stream)))
