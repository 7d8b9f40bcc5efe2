"""CSA2 hot path over an FP4 (E2M1 + E4M3/16) KV cache for AMD MI355X (gfx950).

The compute lives in ``libcsa2.so`` (HIP kernels behind the C ABI in
include/csa2.h); this package is its thin Python binding plus the seeded
synthetic-input module used by tests and the benchmark.
"""
from ._binding import (  # noqa: F401
    BLOCK, POOL_BLOCKS, READ_RATE_SINK_WORDS, SCALE_GROUP, TOPK, WINDOW, EXPORTS, LIB_PATH, AttnArgs, CSA2Error,
    IndexArgs,
    attn_args, attn_workspace_size, check_index, dequantize_kv, index_args, index_full, index_full_append,
    index_full_noalloc,
    index_reindex, index_scan, index_select,
    index_select_append, index_full_append_paged, index_select_append_paged,
    index_workspace_size, load, quantize_kv, quantize_kv_paged, quantize_swa_fp8, read_rate, sparse_attn,
    status_string,
)
from .pipeline import DecodeGroup  # noqa: F401
