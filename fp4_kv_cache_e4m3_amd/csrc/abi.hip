// C ABI of the CSA2 library: host-side validation, workspace sizing and
// dispatch to the gfx950 kernels.  Declarations and contracts: include/csa2.h.
#include <cmath>
#include <cstdlib>
#include <mutex>

#include "../../include/csa2.h"
#include "common.h"
#include "check.h"
#include "quant.h"
#include "rate.h"

// Scratch of csa2_index_full_noalloc: one array per GPU, loaded with the
// library's code object.  Host code never passes this name to a kernel (on
// the host it is only a stand-in); it uses the device address looked up once
// per device below.
__device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

// Debug mode's failure counter (one per GPU; same rule for host code).
__device__ __align__(256) uint32_t debug_bad[64];

namespace {

using namespace csa2;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int64_t kMaxKvLen = 1 << 20;           // 131,072 blocks per query in the pool select
constexpr int64_t kMaxScoreRows = 64 * 65535;    // Qn * H_I: 64 score rows per scan workgroup (32 with fp8)

int check_index(const csa2_index_args* a) {
  if (!a) return CSA2_ERR_NULL;
  if (a->batch < 0 || a->q_per_seq < 1 || a->kv_len < 0 || a->kv_len > kMaxKvLen) return CSA2_ERR_SHAPE;
  if (!(a->heads == 2 || a->heads == 4 || a->heads == 8 || a->heads == 16)) return CSA2_ERR_SHAPE;
  if (!(a->dim == 64 || a->dim == 128)) return CSA2_ERR_SHAPE;
  if ((int64_t)a->q_per_seq * a->heads > (a->fp8 == 1 ? kMaxScoreRows / 2 : kMaxScoreRows)) return CSA2_ERR_SHAPE;
  const int64_t nq = (int64_t)a->batch * a->q_per_seq;
  if (nq > 0 && (!a->q || !a->w)) return CSA2_ERR_NULL;
  if (nq > 0 && a->kv_len > 0 && !a->k) return CSA2_ERR_NULL;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->w, 4)) return CSA2_ERR_ALIGN;
  if (a->fp8 != 0 && a->fp8 != 1) return CSA2_ERR_SHAPE;
  if (a->fp8) {
    if (nq > 0 && !a->q_scale) return CSA2_ERR_NULL;
    if (nq > 0 && a->kv_len > 0 && !a->k_scale) return CSA2_ERR_NULL;
    if (!aligned(a->q_scale, 4) || !aligned(a->k_scale, 4)) return CSA2_ERR_ALIGN;
  }
  return CSA2_OK;
}

// FP8 scale pointers for the kernels: a NULL key-scale pointer selects the
// int8 kernels (with an empty cache both give the same, all-empty, result)
const float* q_scales(const csa2_index_args* a) { return a->fp8 ? a->q_scale : nullptr; }
const float* k_scales(const csa2_index_args* a) { return a->fp8 ? a->k_scale : nullptr; }

// Contexts of at least 2^19 entries take the long path of the Full index:
// the scan writes only the 8-token block maxima, the select forms the pool,
// and the Top-512 comes from rescoring the pool's positions with the layer's
// own indexer query (the Reindex kernels).  That equals the Full layer's
// Top-512 position for position (the pool holds the global Top-512, and the
// rescored keys are the scan's, computed in the same order).  It trades the
// scan's token-key writes (4 B per query and position) for gathers of the
// pool's key rows (2,048 x 8 x D_I bytes per query): cheaper from 2^19
// entries on at D_I = 128.
constexpr int64_t kLongKvLen = 1 << 19;

struct IndexLayout {
  int64_t nq, tk_stride, bk_stride, full_bytes, reindex_bytes, total;
  bool long_path;
  int64_t bk_off, pool_off;          // bytes: block keys; the pool (long path, when the caller passes none)
  int64_t pkeys_off, pthr_off;       // bytes (long path): the pool blocks' keys, the Top-512 key floors
};

IndexLayout index_layout(const csa2_index_args* a) {
  IndexLayout L{};
  L.nq = (int64_t)a->batch * a->q_per_seq;
  L.long_path = a->kv_len >= kLongKvLen;
  L.tk_stride = round_up(a->kv_len, 16);
  L.bk_stride = round_up((a->kv_len + kBlock - 1) / kBlock, 16);
  L.reindex_bytes = L.nq * (kPoolPositions + kPoolBlocks) * 4;     // position keys + block keys
  if (!L.long_path) {
    L.full_bytes = L.nq * (L.tk_stride + L.bk_stride) * 4;
    L.bk_off = L.nq * L.tk_stride * 4;
    L.total = round_up(L.full_bytes > L.reindex_bytes ? L.full_bytes : L.reindex_bytes, 256);
    L.pool_off = L.pkeys_off = L.pthr_off = -1;
  } else {
    // block keys at the front (the Reindex keys reuse that space once the
    // pool is formed), then room for a pool
    L.full_bytes = L.nq * L.bk_stride * 4;
    L.bk_off = 0;
    L.pool_off = round_up(L.full_bytes > L.reindex_bytes ? L.full_bytes : L.reindex_bytes, 256);
    L.pkeys_off = round_up(L.pool_off + L.nq * kPoolBlocks * 4, 256);
    L.pthr_off = L.pkeys_off + L.nq * kPoolBlocks * 4;
    L.total = round_up(L.pthr_off + L.nq * 4, 256);
  }
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// Device address of the current GPU's scratch array, looked up on the first
// call on each device (thread-safe) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return CSA2_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

// ---- debug mode: CSA2_DEBUG=1 when the library is loaded (read once, here)
const bool g_debug = [] {
  const char* v = std::getenv("CSA2_DEBUG");
  return v != nullptr && v[0] == '1' && v[1] == 0;
}();
std::once_flag g_debug_once[kMaxDevices];
uint32_t* g_debug_ptr[kMaxDevices];
hipError_t g_debug_err[kMaxDevices];

// index-row check into `bad` (arguments already validated)
hipError_t check_rows(const csa2_index_args* a, const int32_t* pool, const int32_t* topk, int mode, uint32_t* bad,
                      hipStream_t stream) {
  CheckParams cp{pool, topk, a->n_visible, a->kv_len, mode, bad};
  return launch_check_index(cp, a->batch * a->q_per_seq, stream);
}

// Debug mode after (or, mode 2, before) an index call that returned `st`:
// check the rows on the device, wait for the stream, report failures.
int debug_check(int st, const csa2_index_args* a, const int32_t* pool, const int32_t* topk, int mode,
                hipStream_t stream) {
  if (!g_debug || st != CSA2_OK || (int64_t)a->batch * a->q_per_seq == 0) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_HIP;
  std::call_once(g_debug_once[dev], [dev] {
    void* ptr = nullptr;
    g_debug_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_bad));
    g_debug_ptr[dev] = static_cast<uint32_t*>(ptr);
  });
  if (g_debug_err[dev] != hipSuccess || !g_debug_ptr[dev]) return CSA2_ERR_HIP;
  uint32_t* bad = g_debug_ptr[dev];
  uint32_t host = 0;
  if (hipMemsetAsync(bad, 0, sizeof(uint32_t), stream) != hipSuccess) return CSA2_ERR_HIP;
  if (check_rows(a, pool, topk, mode, bad, stream) != hipSuccess) return CSA2_ERR_HIP;
  if (hipMemcpyAsync(&host, bad, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return host ? CSA2_ERR_DEBUG : CSA2_OK;
}

// Work split of one attention layer.  A workgroup owns (query, 16 heads, one
// column half of the output channels, a contiguous range of 16-entry tiles);
// its NW waves take every NW-th tile.  When the grid fits one workgroup per
// CU (<= 256), 8 waves (two per SIMD) keep the whole tile list in one
// workgroup; otherwise 4-wave workgroups (two per CU) avoid a second wave of
// 8-wave workgroups (384 workgroups at 48 queries: 121 vs 140 us for four
// layers).  Splits of the tile list over workgroups are used only when the
// grid would otherwise leave most CUs idle; their partial states are merged
// by a second kernel.  The caller may fix either choice (csa2_attn_args
// waves / splits; 0 = this choice).
void attn_plan(int64_t nq, int heads, int n_tiles, int want_waves, int want_splits, int& waves, int& splits) {
  const int64_t base = 2 * nq * ((heads + 15) / 16);
  waves = want_waves > 0 ? want_waves : (base <= 256 ? 8 : 4);
  int dflt = 1;
  if (base > 0 && base < 128) {            // fewer than half the CUs busy: split
    dflt = (int)((256 + base - 1) / base);
    const int cap = n_tiles / (2 * waves) > 1 ? n_tiles / (2 * waves) : 1;
    if (dflt > cap) dflt = cap;
  }
  int s = want_splits > 0 ? want_splits : dflt;
  if (n_tiles == 0) s = 1;
  if (s > n_tiles && n_tiles > 0) s = n_tiles;
  const int tps = n_tiles > 0 ? (n_tiles + s - 1) / s : 1;
  splits = n_tiles > 0 ? (n_tiles + tps - 1) / tps : 1;
}

// the prefill kernel (two workgroups per query and 64-head group) pays off
// from about 96 query-head groups on: d = 512, 64 heads, 640 entries per
// query, the decode kernel against it at 64 queries 26.6 vs 33.0 us, at 128
// queries 48.3 vs 35.6 us
constexpr int64_t kWideMinWorkgroups = 96;

struct AttnLayout {
  int64_t nq;
  int n_sparse_tiles, n_tiles, splits, tps, swa_rows, waves;
  bool wide;
  int64_t ws_bytes;
};

AttnLayout attn_layout(const csa2_attn_args* a) {
  AttnLayout L{};
  L.nq = (int64_t)a->batch * a->q_per_seq;
  L.n_sparse_tiles = a->kv_len > 0 ? (a->topk_k + 15) / 16 : 0;
  L.swa_rows = a->window > 0 ? a->window - 1 + a->q_per_seq : 0;
  L.n_tiles = L.n_sparse_tiles + (a->window + 15) / 16;
  const bool wide_ok = a->dim == 512 && a->swa_fp8 == 0 && a->waves == 0 && a->splits == 0 &&
                       !a->topk_rows_out && !a->topk_is_rows;
  L.wide = a->kernel == 2 || (a->kernel == 0 && wide_ok && L.nq * ((a->heads + 63) / 64) >= kWideMinWorkgroups);
  if (L.wide) {
    L.waves = 4;
    L.splits = 1;
    L.tps = L.n_tiles > 0 ? L.n_tiles : 1;
    L.ws_bytes = 0;
    return L;
  }
  attn_plan(L.nq, a->heads, L.n_tiles, a->waves, a->splits, L.waves, L.splits);
  L.tps = L.n_tiles > 0 ? (L.n_tiles + L.splits - 1) / L.splits : 1;
  L.ws_bytes = 0;
  if (L.splits > 1) {
    const int64_t parts = L.nq * L.splits * a->heads;
    L.ws_bytes = round_up(parts * a->dim * 4, 256) + round_up(parts * 2 * 4, 256);
  }
  return L;
}

int check_attn(const csa2_attn_args* a) {
  if (!a) return CSA2_ERR_NULL;
  if (a->batch < 0 || a->q_per_seq < 1 || a->kv_len < 0 || a->kv_len > (int64_t)1 << 31) return CSA2_ERR_SHAPE;
  if (a->heads < 1 || a->heads > 128) return CSA2_ERR_SHAPE;
  if (!(a->waves == 0 || a->waves == 4 || a->waves == 8) || a->splits < 0 || a->splits > 256) return CSA2_ERR_SHAPE;
  if (a->kernel < 0 || a->kernel > 2) return CSA2_ERR_SHAPE;
  if (a->kernel == 2 && (a->dim != 512 || a->swa_fp8 != 0 || a->waves != 0 || a->splits != 0)) return CSA2_ERR_SHAPE;
  if (!(a->dim == 128 || a->dim == 512)) return CSA2_ERR_SHAPE;
  if (a->topk_k < 0 || a->topk_k > kMaxTopK || a->window < 0 || a->window > 1024) return CSA2_ERR_SHAPE;
  const int64_t nq = (int64_t)a->batch * a->q_per_seq;
  if (nq == 0) return CSA2_OK;
  if (nq > 0x7FFFFFF8ll) return CSA2_ERR_SHAPE;
  if (!a->q || !a->out) return CSA2_ERR_NULL;
  if (a->kv_len > 0 && a->topk_k > 0 && (!a->codes || !a->scales || !a->topk)) return CSA2_ERR_NULL;
  if (a->window > 0 && !a->swa) return CSA2_ERR_NULL;
  if (a->swa_fp8 != 0 && a->swa_fp8 != 1) return CSA2_ERR_SHAPE;
  if (a->swa_fp8 && a->window > 0 && !a->swa_scale) return CSA2_ERR_NULL;
  if (a->swa_fp8 && !aligned(a->swa_scale, 4)) return CSA2_ERR_ALIGN;
  if (a->codes_stride < a->dim / 2 || a->scales_stride < a->dim / 16) return CSA2_ERR_SHAPE;
  // one sequence's rows are addressed through 32-bit buffer offsets (24-bit
  // row multiplies)
  constexpr int64_t kBufMax = 0xFFFFE000ll;
  if (a->kv_len >= (1 << 24) || a->codes_stride >= (1 << 24) || a->scales_stride >= (1 << 24) ||
      a->kv_len * a->codes_stride > kBufMax || a->kv_len * a->scales_stride > kBufMax ||
      ((int64_t)a->window - 1 + a->q_per_seq) * a->dim * 2 > kBufMax)
    return CSA2_ERR_SHAPE;
  if (!aligned(a->q, 16) || !aligned(a->codes, 16) || !aligned(a->scales, 8) || !aligned(a->swa, 16) ||
      !aligned(a->out, 16) || !aligned(a->topk, 4) || (a->codes_stride % 16) || (a->scales_stride % 8))
    return CSA2_ERR_ALIGN;
  if (a->block_table) {                              // paged cache: the whole cache is one buffer
    const int ps = a->page_size;
    if (ps < 1 || ps > 65536 || (ps & (ps - 1))) return CSA2_ERR_SHAPE;
    if (a->max_pages < 1 || (int64_t)a->max_pages * ps < a->kv_len) return CSA2_ERR_SHAPE;
    if (a->cache_rows < 0 || a->cache_rows >= (1 << 24) || a->cache_rows * a->codes_stride > kBufMax ||
        a->cache_rows * a->scales_stride > kBufMax)
      return CSA2_ERR_SHAPE;
    if (!aligned(a->block_table, 4)) return CSA2_ERR_ALIGN;
  }
  if (!aligned(a->swa_start, 4)) return CSA2_ERR_ALIGN;
  if (a->swa_new) {                                  // encoded by the attention launch itself
    if (a->swa_fp8 != 1 || a->window < 1 || a->q_per_seq > kMaxSwaNew) return CSA2_ERR_SHAPE;
    if (!aligned(a->swa_new, 16)) return CSA2_ERR_ALIGN;
  }
  // the Top-K as cache rows: written by a paged call, read instead of positions
  if (a->topk_is_rows != 0 && a->topk_is_rows != 1) return CSA2_ERR_SHAPE;
  if ((a->topk_rows_out || a->topk_is_rows) && a->kernel == 2) return CSA2_ERR_SHAPE;
  if (a->topk_rows_out && !a->block_table) return CSA2_ERR_SHAPE;
  if (!aligned(a->topk_rows_out, 4)) return CSA2_ERR_ALIGN;
  if (a->topk_is_rows) {
    if (a->block_table) return CSA2_ERR_SHAPE;
    if (a->cache_rows < 0 || a->cache_rows >= (1 << 24) || a->cache_rows * a->codes_stride > kBufMax ||
        a->cache_rows * a->scales_stride > kBufMax)
      return CSA2_ERR_SHAPE;
  }
  return CSA2_OK;
}

int check_quantize(const float* x, int64_t x_stride, int64_t rows, int32_t dim, const uint8_t* codes,
                   int64_t codes_stride, const uint8_t* scales, int64_t scales_stride) {
  if (rows < 0 || dim < 32 || dim > 4096 || dim % 32) return CSA2_ERR_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_ERR_NULL;
  if (x_stride < dim || codes_stride < dim / 2 || scales_stride < dim / 16) return CSA2_ERR_SHAPE;
  if (!aligned(x, 16) || x_stride % 4 || !aligned(codes, 8) || codes_stride % 8) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

// arguments of the selection stage (and of csa2_index_full before its scan)
int check_select(const csa2_index_args* a, const int32_t* pool, const int32_t* topk, const void* ws,
                 size_t ws_size) {
  int st = check_index(a);
  if (st != CSA2_OK) return st;
  const IndexLayout L = index_layout(a);
  if (L.nq == 0) return CSA2_OK;
  if (!topk) return CSA2_ERR_NULL;
  if (!aligned(a->n_visible, 4) || !aligned(pool, 4) || !aligned(topk, 4)) return CSA2_ERR_ALIGN;
  if (!ws || ws_size < (size_t)L.total || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  return CSA2_OK;
}

// the selection launch, with an optional quantisation job riding along;
// arguments already checked
int select_impl(const csa2_index_args* a, int32_t* pool, int32_t* topk, const void* ws, size_t ws_size,
                const QuantJob& qj, hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  const IndexLayout L = index_layout(a);
  if (L.nq == 0)
    return qj.rows > 0 ? hip_status(launch_quantize(qj.x, qj.xs, qj.rows, 16 * qj.groups, qj.codes, qj.cs, qj.scales,
                                                    qj.ss, stream))
                       : CSA2_OK;
  const uint32_t* tkeys = L.long_path ? nullptr : static_cast<const uint32_t*>(ws);
  const uint32_t* bkeys = reinterpret_cast<const uint32_t*>(static_cast<const char*>(ws) + L.bk_off);
  if (!L.long_path) {
    SelectParams sel{tkeys, L.tk_stride, bkeys, L.bk_stride, a->n_visible, a->kv_len, pool, topk};
    sel.qj = qj;
    return hip_status(launch_select_full(sel, (int)L.nq, (a->kv_len + kBlock - 1) / kBlock, stream));
  }
  // long path: the pool (into the workspace when the caller takes none), then
  // the Top-512 of its positions rescored with this layer's own query
  int32_t* pl = pool ? pool : reinterpret_cast<int32_t*>(static_cast<char*>(const_cast<void*>(ws)) + L.pool_off);
  char* const wsb = static_cast<char*>(const_cast<void*>(ws));
  uint32_t* const pkeys = reinterpret_cast<uint32_t*>(wsb + L.pkeys_off);
  uint32_t* const pthr = reinterpret_cast<uint32_t*>(wsb + L.pthr_off);
  SelectParams sel{nullptr, L.tk_stride, bkeys, L.bk_stride, a->n_visible, a->kv_len, pl, nullptr};
  sel.qj = qj;
  sel.pkeys = pkeys;
  sel.pthr = pthr;
  hipError_t e = launch_select_full(sel, (int)L.nq, (a->kv_len + kBlock - 1) / kBlock, stream);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  // the rescoring gathers only the pool blocks at or above each query's
  // Top-512 key floor (the others hold no Top-512 position)
  uint32_t* rk = reinterpret_cast<uint32_t*>(wsb);
  ReindexParams rp{a->q, a->w, a->k, a->n_visible, q_scales(a), k_scales(a), pl, a->q_per_seq, a->kv_len,
                   rk, topk, rk + L.nq * kPoolPositions, pkeys, pthr};
  return hip_status(launch_reindex(rp, (int)L.nq, a->heads, a->dim, stream));
}

}  // namespace

extern "C" {

const char* csa2_status_string(int s) {
  switch (s) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_NULL: return "CSA2_ERR_NULL: a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "CSA2_ERR_SHAPE: unsupported or inconsistent size";
    case CSA2_ERR_ALIGN: return "CSA2_ERR_ALIGN: pointer or stride misaligned";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE: workspace missing or too small";
    case CSA2_ERR_HIP: return "CSA2_ERR_HIP: the HIP runtime reported an error";
    case CSA2_ERR_SCRATCH:
      return "CSA2_ERR_SCRATCH: the problem needs more than the 64 MiB scratch of csa2_index_full_noalloc";
    case CSA2_ERR_DEBUG:
      return "CSA2_ERR_DEBUG: a pool or Top-K row failed the device-side check (CSA2_DEBUG=1)";
    default: return "unknown csa2 status";
  }
}

int csa2_version(void) { return (1 << 16) | 4; }

int csa2_quantize_kv(const float* x, int64_t x_stride, int64_t rows, int32_t dim, uint8_t* codes,
                     int64_t codes_stride, uint8_t* scales, int64_t scales_stride, hipStream_t stream) {
  const int st = check_quantize(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride);
  if (st != CSA2_OK || rows == 0) return st;
  return hip_status(launch_quantize(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride, stream));
}

int csa2_read_rate(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return CSA2_OK;
  if (!buf || !sink) return CSA2_ERR_NULL;
  if (!aligned(buf, 16) || bytes % 16 || !aligned(sink, 4)) return CSA2_ERR_ALIGN;
  return hip_status(launch_read_rate(buf, (int64_t)bytes, sink, kReadRateWorkgroups, stream));
}

int csa2_quantize_kv_bf16(const uint16_t* x, int64_t x_stride, int64_t rows, int32_t dim, uint8_t* codes,
                          int64_t codes_stride, uint8_t* scales, int64_t scales_stride, hipStream_t stream) {
  // the fp32 checks, with the bf16 row alignment: 16 bytes at x and at every
  // row start (x_stride a multiple of 8 elements)
  if (rows < 0 || dim < 32 || dim > 4096 || dim % 32) return CSA2_ERR_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_ERR_NULL;
  if (x_stride < dim || codes_stride < dim / 2 || scales_stride < dim / 16) return CSA2_ERR_SHAPE;
  if (!aligned(x, 16) || x_stride % 8 || !aligned(codes, 8) || codes_stride % 8) return CSA2_ERR_ALIGN;
  return hip_status(launch_quantize_bf16(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride, stream));
}

// arguments of new rows written through a block table; fills d on success
int check_paged_rows(const float* x, int64_t x_stride, int64_t rows, int32_t dim, const int32_t* row_seq,
                     const int32_t* row_pos, const int32_t* block_table, int32_t batch, int32_t max_pages,
                     int32_t page_size, const uint8_t* codes, int64_t codes_stride, const uint8_t* scales,
                     int64_t scales_stride, int64_t cache_rows, PagedRows& d) {
  int st = check_quantize(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride);
  if (st != CSA2_OK) return st;
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) || max_pages < 1 || batch < 1 ||
      cache_rows < 0 || rows * (dim / 16) > ((int64_t)1 << 28))
    return CSA2_ERR_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!row_seq || !row_pos || !block_table) return CSA2_ERR_NULL;
  if (!aligned(row_seq, 4) || !aligned(row_pos, 4) || !aligned(block_table, 4)) return CSA2_ERR_ALIGN;
  d = PagedRows{row_seq, row_pos, block_table, batch, max_pages, 0, cache_rows};
  while ((1 << d.shift) < page_size) ++d.shift;
  return CSA2_OK;
}

int csa2_quantize_kv_paged(const float* x, int64_t x_stride, int64_t rows, int32_t dim, const int32_t* row_seq,
                           const int32_t* row_pos, const int32_t* block_table, int32_t batch, int32_t max_pages,
                           int32_t page_size, uint8_t* codes, int64_t codes_stride, uint8_t* scales,
                           int64_t scales_stride, int64_t cache_rows, hipStream_t stream) {
  PagedRows d{};
  const int st = check_paged_rows(x, x_stride, rows, dim, row_seq, row_pos, block_table, batch, max_pages, page_size,
                                  codes, codes_stride, scales, scales_stride, cache_rows, d);
  if (st != CSA2_OK || rows == 0) return st;
  return hip_status(launch_quantize_paged(x, x_stride, rows, dim, d, codes, codes_stride, scales, scales_stride,
                                          stream));
}

int csa2_index_select_append_paged(const csa2_index_args* a, int32_t* pool, int32_t* topk, const void* ws,
                                   size_t ws_size, const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                                   const int32_t* row_seq, const int32_t* row_pos, const int32_t* block_table,
                                   int32_t batch, int32_t max_pages, int32_t page_size, uint8_t* codes,
                                   int64_t codes_stride, uint8_t* scales, int64_t scales_stride, int64_t cache_rows,
                                   hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  PagedRows d{};
  st = check_paged_rows(x, x_stride, rows, dim, row_seq, row_pos, block_table, batch, max_pages, page_size, codes,
                        codes_stride, scales, scales_stride, cache_rows, d);
  if (st != CSA2_OK) return st;
  const QuantJob qj{x, x_stride, rows, dim / 16, codes, codes_stride, scales, scales_stride, d};
  return debug_check(select_impl(a, pool, topk, ws, ws_size, qj, stream), a, pool, topk, 0, stream);
}

int csa2_index_full_append_paged(const csa2_index_args* a, int32_t* pool, int32_t* topk, void* ws, size_t ws_size,
                                 const float* x, int64_t x_stride, int64_t rows, int32_t dim, const int32_t* row_seq,
                                 const int32_t* row_pos, const int32_t* block_table, int32_t batch,
                                 int32_t max_pages, int32_t page_size, uint8_t* codes, int64_t codes_stride,
                                 uint8_t* scales, int64_t scales_stride, int64_t cache_rows, hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  PagedRows d{};
  st = check_paged_rows(x, x_stride, rows, dim, row_seq, row_pos, block_table, batch, max_pages, page_size, codes,
                        codes_stride, scales, scales_stride, cache_rows, d);
  if (st != CSA2_OK) return st;
  st = csa2_index_scan(a, ws, ws_size, stream);
  if (st != CSA2_OK) return st;
  const QuantJob qj{x, x_stride, rows, dim / 16, codes, codes_stride, scales, scales_stride, d};
  return debug_check(select_impl(a, pool, topk, ws, ws_size, qj, stream), a, pool, topk, 0, stream);
}

int csa2_quantize_swa_fp8(const uint16_t* x, int64_t x_stride, int64_t rows, int32_t dim, uint8_t* out,
                          int64_t out_stride, float* scales, int64_t scales_stride, hipStream_t stream) {
  if (rows < 0 || dim < 8 || dim > 512 || dim % 8) return CSA2_ERR_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!x || !out || !scales) return CSA2_ERR_NULL;
  if (x_stride < dim || out_stride < dim || scales_stride < 1) return CSA2_ERR_SHAPE;
  if (!aligned(x, 16) || x_stride % 8 || !aligned(out, 8) || out_stride % 8 || !aligned(scales, 4))
    return CSA2_ERR_ALIGN;
  return hip_status(launch_quantize_swa8(x, x_stride, rows, dim, out, out_stride, scales, scales_stride, stream));
}

int csa2_dequantize_kv(const uint8_t* codes, int64_t codes_stride, const uint8_t* scales,
                       int64_t scales_stride, int64_t rows, int32_t dim, float* out, int64_t out_stride,
                       hipStream_t stream) {
  if (rows < 0 || dim < 32 || dim > 4096 || dim % 32) return CSA2_ERR_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!out || !codes || !scales) return CSA2_ERR_NULL;
  if (out_stride < dim || codes_stride < dim / 2 || scales_stride < dim / 16) return CSA2_ERR_SHAPE;
  if (!aligned(out, 16) || out_stride % 4 || !aligned(codes, 8) || codes_stride % 8) return CSA2_ERR_ALIGN;
  return hip_status(launch_dequantize(codes, codes_stride, scales, scales_stride, rows, dim, out, out_stride, stream));
}

size_t csa2_index_workspace_size(const csa2_index_args* a) {
  if (check_index(a) != CSA2_OK) return 0;
  return (size_t)index_layout(a).total;
}

int csa2_index_scan(const csa2_index_args* a, void* ws, size_t ws_size, hipStream_t stream) {
  int st = check_index(a);
  if (st != CSA2_OK) return st;
  const IndexLayout L = index_layout(a);
  if (L.nq == 0) return CSA2_OK;
  if (!aligned(a->n_visible, 4)) return CSA2_ERR_ALIGN;
  if (!ws || ws_size < (size_t)L.total || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  uint32_t* tkeys = L.long_path ? nullptr : static_cast<uint32_t*>(ws);
  uint32_t* bkeys = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.bk_off);
  ScanParams sp{a->q, a->w, a->k, a->n_visible, q_scales(a), k_scales(a), a->batch, a->q_per_seq, a->kv_len,
                tkeys, L.tk_stride, bkeys, L.bk_stride};
  return hip_status(launch_index_scan(sp, a->heads, a->dim, stream));
}

int csa2_index_select(const csa2_index_args* a, int32_t* pool, int32_t* topk, const void* ws,
                      size_t ws_size, hipStream_t stream) {
  return debug_check(select_impl(a, pool, topk, ws, ws_size, QuantJob{}, stream), a, pool, topk, 0, stream);
}

int csa2_index_full(const csa2_index_args* a, int32_t* pool, int32_t* topk, void* ws, size_t ws_size,
                    hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  st = csa2_index_scan(a, ws, ws_size, stream);
  if (st != CSA2_OK) return st;
  return debug_check(select_impl(a, pool, topk, ws, ws_size, QuantJob{}, stream), a, pool, topk, 0, stream);
}

int csa2_index_full_noalloc(const csa2_index_args* a, int32_t* pool, int32_t* topk, hipStream_t stream) {
  int st = check_index(a);
  if (st != CSA2_OK) return st;
  const IndexLayout L = index_layout(a);
  if ((size_t)L.total > CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_ERR_SCRATCH;
  if (L.nq == 0) return CSA2_OK;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != CSA2_OK) return st;
  return csa2_index_full(a, pool, topk, ws, CSA2_NOALLOC_SCRATCH_BYTES, stream);
}

int csa2_index_select_append(const csa2_index_args* a, int32_t* pool, int32_t* topk, const void* ws,
                             size_t ws_size, const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                             uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                             hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  st = check_quantize(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride);
  if (st != CSA2_OK) return st;
  const QuantJob qj{x, x_stride, rows, dim / 16, codes, codes_stride, scales, scales_stride};
  return debug_check(select_impl(a, pool, topk, ws, ws_size, qj, stream), a, pool, topk, 0, stream);
}

int csa2_index_full_append(const csa2_index_args* a, int32_t* pool, int32_t* topk, void* ws, size_t ws_size,
                           const float* x, int64_t x_stride, int64_t rows, int32_t dim, uint8_t* codes,
                           int64_t codes_stride, uint8_t* scales, int64_t scales_stride, hipStream_t stream) {
  int st = check_select(a, pool, topk, ws, ws_size);
  if (st != CSA2_OK) return st;
  st = check_quantize(x, x_stride, rows, dim, codes, codes_stride, scales, scales_stride);
  if (st != CSA2_OK) return st;
  st = csa2_index_scan(a, ws, ws_size, stream);
  if (st != CSA2_OK) return st;
  const QuantJob qj{x, x_stride, rows, dim / 16, codes, codes_stride, scales, scales_stride};
  return debug_check(select_impl(a, pool, topk, ws, ws_size, qj, stream), a, pool, topk, 0, stream);
}

int csa2_index_reindex(const csa2_index_args* a, const int32_t* pool, int32_t* topk, void* ws,
                       size_t ws_size, hipStream_t stream) {
  int st = check_index(a);
  if (st != CSA2_OK) return st;
  const IndexLayout L = index_layout(a);
  if (L.nq == 0) return CSA2_OK;
  if (!topk || !pool) return CSA2_ERR_NULL;
  if (!aligned(a->n_visible, 4) || !aligned(pool, 4)) return CSA2_ERR_ALIGN;
  if (!ws || ws_size < (size_t)L.total || !aligned(ws, 256)) return CSA2_ERR_WORKSPACE;
  st = debug_check(CSA2_OK, a, pool, nullptr, 2, stream);   // debug mode: the pool's shape first
  if (st != CSA2_OK) return st;
  ReindexParams rp{a->q, a->w, a->k, a->n_visible, q_scales(a), k_scales(a), pool, a->q_per_seq, a->kv_len,
                   static_cast<uint32_t*>(ws), topk,
                   static_cast<uint32_t*>(ws) + L.nq * kPoolPositions};
  return debug_check(hip_status(launch_reindex(rp, (int)L.nq, a->heads, a->dim, stream)), a, pool, topk, 1, stream);
}

int csa2_check_index(const csa2_index_args* a, const int32_t* pool, const int32_t* topk, int32_t mode, uint32_t* bad,
                     hipStream_t stream) {
  int st = check_index(a);
  if (st != CSA2_OK) return st;
  if (mode < 0 || mode > 2) return CSA2_ERR_SHAPE;
  if ((int64_t)a->batch * a->q_per_seq == 0) return CSA2_OK;
  if (!bad || (mode != 2 && !topk) || (mode != 0 && !pool)) return CSA2_ERR_NULL;
  if (!aligned(bad, 4) || !aligned(pool, 4) || !aligned(topk, 4) || !aligned(a->n_visible, 4)) return CSA2_ERR_ALIGN;
  return hip_status(check_rows(a, pool, mode == 2 ? nullptr : topk, (int)mode, bad, stream));
}

size_t csa2_attn_workspace_size(const csa2_attn_args* a) {
  if (check_attn(a) != CSA2_OK) return 0;
  return (size_t)attn_layout(a).ws_bytes;
}

int csa2_sparse_attn(const csa2_attn_args* a, void* ws, size_t ws_size, hipStream_t stream) {
  int st = check_attn(a);
  if (st != CSA2_OK) return st;
  const AttnLayout L = attn_layout(a);
  if (L.nq == 0) return CSA2_OK;
  if (L.ws_bytes > 0 && (!ws || ws_size < (size_t)L.ws_bytes || !aligned(ws, 256))) return CSA2_ERR_WORKSPACE;
  if (!aligned(a->swa_len, 4)) return CSA2_ERR_ALIGN;
  AttnParams p{};
  p.q = a->q; p.codes = a->codes; p.scales = a->scales; p.topk = a->topk; p.swa = a->swa;
  p.swa_len = a->swa_len; p.out = a->out;
  p.opart = static_cast<float*>(ws);
  p.mlpart = L.ws_bytes > 0 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                         round_up(L.nq * L.splits * a->heads * a->dim * 4, 256))
                            : nullptr;
  p.T = a->kv_len; p.codes_stride = a->codes_stride; p.scales_stride = a->scales_stride; p.nq = L.nq;
  p.qn_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == a->q_per_seq) p.qn_shift = sh;
  p.qn = a->q_per_seq; p.heads = a->heads; p.topk_k = a->topk_k; p.window = a->window;
  p.swa_rows = L.swa_rows; p.splits = L.splits; p.tiles_per_split = L.tps;
  p.n_sparse_tiles = L.n_sparse_tiles; p.n_tiles = L.n_tiles;
  const float sm = a->sm_scale > 0.0f ? a->sm_scale : 1.0f / std::sqrt((float)a->dim);
  p.qscale = sm * 1.4426950408889634f;
  p.swa_fp8 = a->swa_fp8;
  p.swa_scale = a->swa_scale;
  p.block_table = a->block_table;
  if (a->block_table) {
    p.max_pages = a->max_pages;
    p.page_shift = 0;
    while ((1 << p.page_shift) < a->page_size) ++p.page_shift;
    p.cache_rows = a->cache_rows;
  }
  p.swa_start = a->swa_start;
  p.swa_new = a->swa_new;
  p.rows_out = a->topk_rows_out;
  p.rows_in = a->topk_is_rows;
  if (a->topk_is_rows) p.cache_rows = a->cache_rows;
  // With no tile at all the kernel still runs: every head ends with an empty
  // softmax and writes zeros (no memset node, so the call stays graph-safe).
  if (L.wide) return hip_status(launch_attn_wide(p, (int)L.nq, stream));
  return hip_status(launch_attn(p, (int)L.nq, a->dim, L.waves, stream));
}

}  // extern "C"
