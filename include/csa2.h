/*
 * csa2.h -- C ABI of the CSA2 hot path over an FP4 (E2M1 + E4M3/16) KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: DeepSeek-V4.1-Flash pages.
 *   - Layer modes Full / Reindex / Reuse and the hierarchical indexer
 *     (candidate pool of 2,048 blocks x 8 tokens = 16,384 positions, fresh
 *     Top-512): ai-maestro.online, section "Compressed Sparse Attention 2";
 *     wpnews.pro, "What is Compressed Sparse Attention 2 CSA2?".
 *   - FP4 main KV: E2M1 codes with one E4M3 scale per 16 channels, NVFP4
 *     without its global scale: ai-maestro.online, "FP4 KV, Bounded Replay,
 *     and other extensions".
 *   - 128-token sliding window in every layer, own Q and SWA cache per layer:
 *     ai-maestro.online, "Causal Encoder-Decoder architecture" and
 *     "Compressed Sparse Attention 2".
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates device memory and never synchronises the host.
 *   - Work is enqueued on `stream` (NULL = the default stream) and runs
 *     asynchronously; outputs are valid once the stream reaches that point.
 *   - Arguments are validated on the host first.  On any error nothing is
 *     launched and no output or workspace byte is written.  CSA2_ERR_HIP is
 *     returned when the HIP runtime rejects a launch (hipGetLastError).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Calls that share a workspace must be ordered on one stream; calls with
 *     distinct workspaces may run concurrently.
 *   - Reuse layers have no entry point: they pass the latest Top-K buffer to
 *     csa2_sparse_attn (ai-maestro.online, "Compressed Sparse Attention 2":
 *     Reuse skips the indexer entirely).
 *   - Debug mode: with CSA2_DEBUG=1 in the environment when the library is
 *     loaded (read once, at load), every index call checks its pool and
 *     Top-K rows on the device after its launches (csa2_check_index, mode 0
 *     or 1), csa2_index_reindex first checks the shape of the pool it is
 *     given (mode 2), and the call then synchronises its stream and returns
 *     CSA2_ERR_DEBUG when a row fails.  Debug mode breaks the
 *     no-synchronisation rule above and is off by default.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_TOPK 512          /* fresh Top-512 per query token              */
#define CSA2_BLOCK 8           /* tokens per indexer block                   */
#define CSA2_POOL_BLOCKS 2048  /* blocks in the Full layer's candidate pool  */
#define CSA2_WINDOW 128        /* sliding-window rows per query              */
#define CSA2_SCALE_GROUP 16    /* channels sharing one E4M3 scale            */

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,       /* a required pointer is NULL                     */
  CSA2_ERR_SHAPE = 2,      /* unsupported or inconsistent size               */
  CSA2_ERR_ALIGN = 3,      /* pointer or stride not aligned as documented    */
  CSA2_ERR_WORKSPACE = 4,  /* workspace NULL or smaller than the query says  */
  CSA2_ERR_HIP = 5,        /* the HIP runtime reported a launch error        */
  CSA2_ERR_SCRATCH = 6,    /* csa2_index_full_noalloc: the problem needs more
                              than its fixed scratch (CSA2_NOALLOC_SCRATCH_BYTES) */
  CSA2_ERR_DEBUG = 7       /* debug mode (CSA2_DEBUG=1): a pool or Top-K row
                              failed the device-side check (csa2_check_index) */
} csa2_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* csa2_status_string(int status);

/* ABI version, (major << 16) | minor. */
int csa2_version(void);

/*
 * csa2_read_rate -- reads every byte of buf once (16-byte non-temporal loads,
 * one contiguous chunk per workgroup, 16,384 workgroups) and writes one word
 * per wave to sink.  Not a step
 * of the method: timing it with events gives the device's achievable HBM
 * read rate, the reference beside the 8 TB/s peak for the streaming kernels.
 *   buf    device, 16-byte aligned; bytes a multiple of 16 (0: no-op).
 *   sink   device uint32 [CSA2_READ_RATE_SINK_WORDS], 4-byte aligned; its
 *          contents are XORs of the data, with no meaning.
 * Errors: CSA2_ERR_NULL (buf or sink NULL), CSA2_ERR_ALIGN; nothing launched.
 */
#define CSA2_READ_RATE_SINK_WORDS 65536
int csa2_read_rate(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * csa2_quantize_kv -- FP4 quantisation of main-KV rows.
 * Source: ai-maestro.online, "FP4 KV, Bounded Replay, and other extensions".
 *
 * For every row r < rows and every 16-channel group g of x[r, 0:dim):
 *   amax  = max |x|;  scale = E4M3(amax / 6), round to nearest, ties to the
 *   even code, saturating at 448 (code 0x7E), never NaN;
 *   code_i = E2M1(x_i / scale), nearest, ties to even, saturating at 6, sign
 *   bit = sign bit of x_i; a zero scale gives signed-zero codes.
 * Both roundings are decided exactly (threshold compares, no rounded
 * quotient), so the result equals the exact-arithmetic definition.
 *
 *   x           fp32, row r at x + r * x_stride (elements); 16-byte aligned,
 *               x_stride % 4 == 0.  Finite inputs; NaN/Inf give unspecified
 *               (but deterministic) codes.
 *   rows        >= 0 (0 is a no-op).
 *   dim         % 32 == 0, 32 .. 4096.
 *   codes       out, row r at codes + r * codes_stride (bytes): dim/2 bytes,
 *               byte j = code[2j] | code[2j+1] << 4.  8-byte aligned,
 *               codes_stride % 8 == 0, codes_stride >= dim/2.
 *   scales      out, row r at scales + r * scales_stride: dim/16 E4M3FN bytes.
 *               scales_stride >= dim/16.
 * Strided rows let the caller write new tokens straight into their slots of
 * a [B, T] cache (row stride T * row bytes).
 */
int csa2_quantize_kv(const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                     uint8_t* codes, int64_t codes_stride,
                     uint8_t* scales, int64_t scales_stride, hipStream_t stream);

/*
 * csa2_quantize_kv_bf16 -- csa2_quantize_kv for bf16 rows (the same passage:
 * ai-maestro.online, "FP4 KV, Bounded Replay, and other extensions").
 * Every bf16 value widens exactly to fp32, and the codes and scales are
 * exactly those csa2_quantize_kv writes for the widened rows.
 *
 *   x           bf16 bit patterns, row r at x + r * x_stride (elements);
 *               16-byte aligned, x_stride % 8 == 0.
 *   rows, dim, codes, codes_stride, scales, scales_stride, stream: as above.
 * Errors as csa2_quantize_kv (CSA2_ERR_ALIGN for the bf16 alignment above).
 */
int csa2_quantize_kv_bf16(const uint16_t* x, int64_t x_stride, int64_t rows, int32_t dim,
                          uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                          hipStream_t stream);

/*
 * csa2_quantize_kv_paged -- csa2_quantize_kv of new rows into a paged cache.
 * The quantisation happens where the row is written, as for the contiguous
 * cache (wpnews.pro TL;DR: the FP4 cache needs no separate quantisation
 * pass); only the destination differs.  Row r of x (the token at position
 * row_pos[r] of sequence row_seq[r]) is written to cache row
 *     block_table[row_seq[r] * max_pages + row_pos[r] / page_size] * page_size
 *         + row_pos[r] % page_size
 * of codes / scales (same row format as csa2_quantize_kv).  Rows whose
 * sequence is outside [0, batch), whose position is negative or past
 * max_pages * page_size, whose page id is negative or whose cache row is at
 * or past cache_rows are skipped.  Destination rows must be distinct.
 *   row_seq, row_pos  int32 [rows] device arrays, 4-byte aligned.
 *   block_table       int32 [batch, max_pages], 4-byte aligned.
 *   page_size         power of two, 1 .. 65536.
 *   rows * dim / 16 <= 2^28.
 */
int csa2_quantize_kv_paged(const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                           const int32_t* row_seq, const int32_t* row_pos,
                           const int32_t* block_table, int32_t batch, int32_t max_pages, int32_t page_size,
                           uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                           int64_t cache_rows, hipStream_t stream);

/*
 * csa2_quantize_swa_fp8 -- 8-bit sliding-window rows.
 * Source: kongchang.com, "Three Core Innovations" (the window keeps 8-bit
 * precision); the format is not given on the pages.  Each bf16 row r < rows
 * of dim channels becomes E4M3FN codes with one power-of-two scale:
 *   scale = 2^k, k the smallest integer with max|x| <= 448 * 2^k (1 for an
 *   all-zero row);  code_i = E4M3(|x_i| / scale) to nearest, ties to the
 *   even code, sign bit = sign bit of x_i.
 * The division is exact and the rounding is decided exactly.
 *   x       bf16 bits, row r at x + r * x_stride (elements); 16-byte aligned,
 *           x_stride % 8 == 0.
 *   dim     % 8 == 0, 8 .. 512.
 *   out     E4M3 codes, row r at out + r * out_stride (bytes); 8-byte aligned,
 *           out_stride % 8 == 0, out_stride >= dim.
 *   scales  fp32, row r's scale at scales[r * scales_stride]; 4-byte aligned,
 *           scales_stride >= 1 (strided rows let a decode step write its new
 *           row straight into the newest slot of every sequence's window).
 * csa2_sparse_attn reads such rows as its window when swa_fp8 is set.
 */
int csa2_quantize_swa_fp8(const uint16_t* x, int64_t x_stride, int64_t rows, int32_t dim,
                          uint8_t* out, int64_t out_stride, float* scales, int64_t scales_stride,
                          hipStream_t stream);

/*
 * csa2_dequantize_kv -- values of FP4 rows as fp32 (code value x E4M3 scale,
 * exact).  Same row layout and alignment as csa2_quantize_kv; out is fp32
 * [rows, dim] at out + r * out_stride (elements), 16-byte aligned,
 * out_stride % 4 == 0.  Uses the same device decoder as csa2_sparse_attn.
 */
int csa2_dequantize_kv(const uint8_t* codes, int64_t codes_stride,
                       const uint8_t* scales, int64_t scales_stride,
                       int64_t rows, int32_t dim, float* out, int64_t out_stride,
                       hipStream_t stream);

/*
 * Indexer arguments (Full and Reindex layers).
 * Source: ai-maestro.online, "Compressed Sparse Attention 2".
 * The pages do not print the score; the library computes, per query q and
 * visible position t,
 *     s(q, t) = sum_h w[q, h] * max(0, sum_c iq[q, h, c] * ik[b, t, c])
 * with b = q / q_per_seq, the dot products in exact int32 and the weighted
 * sum in fp32 (heads in ascending order).  Scores are exact whenever w is
 * integer-valued and all partial sums stay below 2^24.  Ranking is by
 * (score descending, position ascending): ties go to the lower position.
 *
 * Real-valued indexer (fp8 = 1; the pages leave the indexer's precision
 * open): q and k hold OCP E4M3FN codes, q_scale one fp32 scale per (query,
 * head) and k_scale one per key position, and
 *     s(q, t) = sum_h w[q, h] * max(0, q_scale[q, h] * k_scale[b, t] *
 *                                      sum_c E4M3(q[q, h, c]) * E4M3(k[b, t, c])),
 * evaluated in fp32 as k_scale[b, t] * sum_h (w[q, h] * q_scale[q, h]) *
 * max(0, dot), the dot products summing exact products with fp32
 * accumulation (codes decoded exactly to fp16, fp16 MFMA).  Scales must be
 * positive and finite; NaN codes (0x7F, 0xFF)
 * give unspecified rankings.  The result differs from the exact score by at
 * most (D_I + H_I + 4) * 2^-24 times sum_h |w| q_scale k_scale sum_c |q_c k_c|,
 * so two positions closer than that may rank in either order.
 */
typedef struct {
  int32_t batch;             /* B sequences                                   */
  int32_t q_per_seq;         /* Qn query tokens per sequence; nq = B * Qn    */
  int64_t kv_len;            /* T rows per sequence in ik (row b * T + t)     */
  int32_t heads;             /* H_I: 2, 4, 8 or 16                            */
  int32_t dim;               /* D_I: 64 or 128                                */
  const int8_t* q;           /* iq [nq, H_I, D_I], 16-byte aligned            */
  const float* w;            /* iw [nq, H_I]                                  */
  const int8_t* k;           /* ik [B, T, D_I] contiguous, 16-byte aligned    */
  const int32_t* n_visible;  /* [nq] in [0, T] or NULL (= T): query q sees
                                positions [0, n_visible[q])                  */
  int32_t fp8;               /* 0: int8 q and k.  1: E4M3FN codes + scales   */
  const float* q_scale;      /* fp8: [nq, H_I] fp32 > 0, 4-byte aligned       */
  const float* k_scale;      /* fp8: [B, T] fp32 > 0 (row b * T + t), 4-byte
                                aligned; both NULL when fp8 == 0              */
} csa2_index_args;

/* Bytes of workspace csa2_index_full / csa2_index_reindex need (0 on bad args). */
size_t csa2_index_workspace_size(const csa2_index_args* args);

/*
 * csa2_index_full -- Full layer: score every visible position, take each
 * 8-token block's maximum (blocks aligned at position 0; a partial block
 * uses its visible positions), keep the top min(2048, #blocks) blocks by
 * (block score desc, block id asc) as the pool, and select the top
 * min(512, #pool positions) pool positions by (score desc, position asc).
 * This equals the Top-512 over all visible positions.
 *   pool   out [nq, 2048] int32 block ids, ascending, padded with -1
 *          (may be NULL when no Reindex layer will consume it).
 *   topk   out [nq, 512] int32 positions, ascending, padded with -1.
 *   ws     workspace of csa2_index_workspace_size(args) bytes, 256-B aligned.
 * Supports Qn * H_I <= 4,194,240 (prefill chunks included; 2,097,120 with
 * fp8).
 */
int csa2_index_full(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                    void* ws, size_t ws_size, hipStream_t stream);

/*
 * csa2_index_full_noalloc -- csa2_index_full for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace; the scan's score
 * and block keys go to a fixed scratch array of CSA2_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends
 * (its address is looked up once per device on the first call there).  The
 * call allocates nothing.  Sizes whose csa2_index_workspace_size exceeds the
 * scratch return CSA2_ERR_SCRATCH before any launch.  Every call on one GPU
 * shares that GPU's scratch: calls that may overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller.
 * Results are those of csa2_index_full, bit for bit.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int csa2_index_full_noalloc(const csa2_index_args* args, int32_t* pool, int32_t* topk, hipStream_t stream);

/*
 * The two stages of csa2_index_full, for callers that schedule them apart
 * (e.g. to time or overlap the scan).  csa2_index_scan streams the indexer
 * keys once and writes every visible position's score key and every 8-token
 * block's maximum into `ws`; csa2_index_select then forms the pool and the
 * Top-512 from that workspace.  Both must get the same `args` and `ws`, in
 * this order on one stream; together they equal csa2_index_full.
 */
int csa2_index_scan(const csa2_index_args* args, void* ws, size_t ws_size, hipStream_t stream);
int csa2_index_select(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                      const void* ws, size_t ws_size, hipStream_t stream);

/*
 * csa2_index_full_append / csa2_index_select_append -- csa2_index_full
 * (resp. csa2_index_select) together with csa2_quantize_kv of the step's new
 * main-KV rows (x, x_stride, rows, dim, codes, codes_stride, scales,
 * scales_stride: exactly as csa2_quantize_kv).  A Full layer writes its own
 * entries into the FP4 cache as it indexes (ai-maestro.online, "FP4 KV,
 * Bounded Replay, and other extensions": quantisation happens where the KV
 * is written); the rows are independent of the indexer, so a small job
 * (rows * dim / 16 <= 8,192 groups) runs as extra workgroups of the
 * selection launch instead of a launch of its own; a larger one is launched
 * before the selection.  Results are identical to the separate calls.  All
 * arguments are validated before anything is launched; on error nothing is
 * written.  The new rows must not be read by anything the call itself reads
 * (the indexer never reads the main KV).
 */
int csa2_index_full_append(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                           void* ws, size_t ws_size,
                           const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                           uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                           hipStream_t stream);
int csa2_index_select_append(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                             const void* ws, size_t ws_size,
                             const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                             uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                             hipStream_t stream);

/*
 * csa2_index_full_append_paged / csa2_index_select_append_paged --
 * csa2_index_full_append / csa2_index_select_append with the new rows
 * written into a paged cache as csa2_quantize_kv_paged writes them (same
 * arguments, same skipping rules), as extra workgroups of the selection
 * launch.  Everything is validated before anything is launched.
 */
int csa2_index_full_append_paged(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                                 void* ws, size_t ws_size,
                                 const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                                 const int32_t* row_seq, const int32_t* row_pos,
                                 const int32_t* block_table, int32_t batch, int32_t max_pages, int32_t page_size,
                                 uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                                 int64_t cache_rows, hipStream_t stream);
int csa2_index_select_append_paged(const csa2_index_args* args, int32_t* pool, int32_t* topk,
                                   const void* ws, size_t ws_size,
                                   const float* x, int64_t x_stride, int64_t rows, int32_t dim,
                                   const int32_t* row_seq, const int32_t* row_pos,
                                   const int32_t* block_table, int32_t batch, int32_t max_pages, int32_t page_size,
                                   uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                                   int64_t cache_rows, hipStream_t stream);

/*
 * csa2_index_reindex -- Reindex layer: rescore only the positions of the last
 * Full layer's pool with this layer's own iq / iw and select the top
 * min(512, #positions) by (score desc, position asc).
 *   pool   in [nq, 2048] block ids as written by csa2_index_full for the
 *          same query tokens: ascending, -1 only as trailing padding.
 *          Ids outside [0, ceil(T/8)) are treated as empty.
 *   topk   out [nq, 512], ascending, padded with -1.
 */
int csa2_index_reindex(const csa2_index_args* args, const int32_t* pool, int32_t* topk,
                       void* ws, size_t ws_size, hipStream_t stream);

/*
 * csa2_check_index -- device-side check of index rows against the contract
 * the calls above follow (ai-maestro.online, "Compressed Sparse Attention 2":
 * a pool of 2,048 eight-token blocks, a fresh Top-512 taken from it;
 * Reindex rescores the Full layer's pool of the same query tokens), one
 * workgroup per query.  For query q with n = n_visible[q] (T when NULL):
 *   mode 0 (Full outputs): pool (may be NULL) holds exactly min(2048,
 *          ceil(n/8)) block ids, strictly ascending, in [0, ceil(n/8)), then
 *          -1; topk holds exactly min(512, n) positions, strictly ascending,
 *          in [0, n) and inside pool blocks (when pool is given), then -1.
 *   mode 1 (Reindex outputs, pool = its input): topk holds min(512, p)
 *          positions (p = positions of the pool's blocks below n, the pool's
 *          ids outside [0, ceil(n/8)) counting as empty), strictly
 *          ascending, in [0, n) and inside pool blocks, then -1.
 *   mode 2 (a Reindex input pool): ids >= 0 strictly ascending, then -1.
 * pool, topk: device int32 [nq, 2048] / [nq, 512] as the calls above take
 * them (topk unused in mode 2; pool required in modes 1 and 2).  bad: device
 * uint32; the number of failing rows (a query counts once for its pool and
 * once for its Top-K row) is added to *bad, which the caller zeroes.  args
 * supplies nq, T and n_visible and must pass the same checks as the index
 * calls.  All buffers stay the caller's; only *bad is written, on `stream`,
 * with no wait.  Errors (nothing launched): CSA2_ERR_SHAPE for a mode outside
 * 0..2 or arguments the index calls reject, CSA2_ERR_NULL for a missing
 * buffer the mode needs, CSA2_ERR_ALIGN for a pointer not 4-byte aligned.
 * No queries (batch x q_per_seq = 0): CSA2_OK, nothing launched.
 */
int csa2_check_index(const csa2_index_args* args, const int32_t* pool, const int32_t* topk, int32_t mode,
                     uint32_t* bad, hipStream_t stream);

/*
 * Sparse + sliding-window attention of one CSA2 layer.
 * Source: ai-maestro.online, "Compressed Sparse Attention 2" (own main Q and
 * SWA cache per layer; Top-K indices from the Full/Reindex layer) and
 * "Causal Encoder-Decoder architecture" (128-token window).
 * For query q (sequence b = q / Qn, index j = q % Qn) and head h:
 *   entries = { FP4 row b*T + t : t in topk[q], 0 <= t < T }  followed by
 *             { swa[b, r] : j <= r < j + window, r >= swa_rows - swa_len[b] },
 *   out[q, h] = sum_e softmax_e(sm_scale * Q[q,h] . e) * e   (key = value)
 * in one softmax; a query with no entry gets zeros.
 * Arithmetic (fp32 accumulation throughout): the FP4 entries' logits run on
 * fp16 MFMA (FP4 values are exact in fp16) against Q converted bf16 -> fp16,
 * exact for magnitudes in [2^-14, 65504] (smaller ones lose at most 2^-25
 * absolute); bf16 window entries' logits run on bf16 MFMA against Q and the
 * rows as given (exact products), 8-bit ones on fp16 MFMA like the FP4
 * entries.  sm_scale is applied to the fp32 logits,
 * probabilities are rounded to fp16 and normalised by the sum of the rounded
 * values, and PV runs on fp16 MFMA with the window rows converted to fp16 as
 * Q is.  Requires |Q| and |SWA| below 65504.
 */
typedef struct {
  int32_t batch;               /* B                                            */
  int32_t q_per_seq;           /* Qn; nq = B * Qn                              */
  int64_t kv_len;              /* T rows per sequence in the FP4 cache, < 2^24;
                                  T * codes_stride and T * scales_stride must
                                  stay below 4 GiB - 8 KiB                      */
  int32_t heads;               /* H: 1 .. 128 (a workgroup takes 16 heads; a
                                  last partial group reads zero Q rows)        */
  int32_t dim;                 /* d: 128 or 512                                */
  const uint16_t* q;           /* bf16 [nq, H, d], 16-byte aligned             */
  const uint8_t* codes;        /* FP4 codes, row b*T+t at codes + row*codes_stride;
                                  16-byte aligned rows                         */
  int64_t codes_stride;        /* bytes, % 16 == 0, >= d/2                     */
  const uint8_t* scales;       /* E4M3 scales, row at scales + row*scales_stride */
  int64_t scales_stride;       /* bytes, % 8 == 0, >= d/16                     */
  const int32_t* topk;         /* [nq, topk_k] positions, -1 = empty           */
  int32_t topk_k;              /* entries per Top-K row, 0 .. 2048             */
  const uint16_t* swa;         /* bf16 [B, swa_rows, d], swa_rows = window-1+Qn */
  int32_t window;              /* 0 .. 1024 (128 on the pages)                 */
  const int32_t* swa_len;      /* [B] valid trailing SWA rows, or NULL (= all) */
  float sm_scale;              /* <= 0 selects 1/sqrt(d)                       */
  float* out;                  /* fp32 [nq, H, d]                              */
  int32_t swa_fp8;             /* 0: swa is bf16 as above.  1: swa holds E4M3
                                  codes [B, swa_rows, d] (bytes; rows as written
                                  by csa2_quantize_swa_fp8) and swa_scale their
                                  row scales; a window value is E4M3(code) *
                                  scale, exact in fp16 when every row scale is
                                  in [2^-15, 2^7]                              */
  const float* swa_scale;      /* fp32 [B, swa_rows] powers of two (swa_fp8)   */
  /* Paged FP4 cache (block_table != NULL): codes / scales hold cache_rows
     physical rows in pages of page_size rows; position t of sequence b is
     row block_table[b * max_pages + t / page_size] * page_size
         + t % page_size.
     A negative page id, or a row at or past cache_rows, leaves that Top-K
     entry empty.  The same stride and alignment rules apply; a row may be
     shared by several sequences.  NULL: the contiguous [B, T] layout above. */
  const int32_t* block_table;  /* [B, max_pages] int32, 4-byte aligned        */
  int32_t max_pages;           /* >= ceil(T / page_size)                       */
  int32_t page_size;           /* power of two, 1 .. 65536                     */
  int64_t cache_rows;          /* < 2^24; cache_rows * codes_stride and
                                  cache_rows * scales_stride < 4 GiB - 8 KiB   */
  /* Window ring buffer: NULL, or [B] int32 start slots.  Window row r of
     sequence b (the r of the window description above) is stored in slot
     (swa_start[b] + r) mod swa_rows of that sequence's swa (and swa_scale)
     rows, so a decode step overwrites one slot instead of shifting the
     window.  Starts outside [0, swa_rows) count as 0.  */
  const int32_t* swa_start;
  /* Work split (0 = the library's choice for the shape).  waves: 4 or 8
     waves per workgroup, each taking every waves-th 16-entry tile of its
     query; splits >= 1: the tile list is cut into that many contiguous
     ranges, one workgroup each, whose partial softmax states a second kernel
     merges (needs csa2_attn_workspace_size bytes of workspace).  Both change
     the fp32 summation order, so outputs may differ in the last bits between
     choices; each choice is deterministic.  Other values: CSA2_ERR_SHAPE.   */
  int32_t waves;
  int32_t splits;
  /* Kernel: 0 = the library's choice; 1 = workgroups of 16 heads (waves and
     splits above apply); 2 = two workgroups per query and 64 heads (one per
     32 heads), for many query tokens at once (a prefill chunk): each FP4 row
     is decoded twice per query instead of once per 16 heads, and the logits
     once; needs dim = 512, swa_fp8 = 0 and waves = splits = 0.  The
     library's choice is 2 where that holds and nq * ceil(H / 64) >= 96,
     else 1.  The kernels
     sum in different orders (results may differ in the last bits); each is
     deterministic.  Other values: CSA2_ERR_SHAPE.                            */
  int32_t kernel;
  /* 8-bit windows (swa_fp8 = 1, window >= 1) only: NULL, or the step's new
     window rows as bf16 [nq, d], 16-byte aligned, Qn <= 16.  Row b * Qn + i
     is window row swa_rows - Qn + i of sequence b (the step's query
     tokens).  The call encodes each exactly as csa2_quantize_swa_fp8 does,
     attends over the encoded values, and stores the codes and the row scale
     into swa and swa_scale at that row (its ring slot when swa_start is
     given), so both must be writable; their previous contents at those rows
     are not read.  This replaces a csa2_quantize_swa_fp8 launch per layer and
     step.  Errors: CSA2_ERR_SHAPE (bf16 window, no window, Qn > 16),
     CSA2_ERR_ALIGN.                                                        */
  const uint16_t* swa_new;
  /* Top-K as cache rows, for the later layers of a group over a paged cache:
     topk_rows_out (block_table given): NULL, or int32 [nq, topk_k], 4-byte
     aligned; the call also writes each Top-K slot's cache row there (-1 for
     an empty slot, a position outside [0, T), a negative page id or a row at
     or past cache_rows).  topk_is_rows = 1 (block_table NULL): topk holds
     such rows, codes / scales span cache_rows rows as for a paged cache and
     a row outside [0, cache_rows) leaves its slot empty; the result equals
     the paged call that wrote them, without its block-table reads.  Both
     need kernel 0 or 1 (the library then takes 1).  Errors: CSA2_ERR_SHAPE,
     CSA2_ERR_ALIGN.                                                        */
  int32_t* topk_rows_out;
  int32_t topk_is_rows;
} csa2_attn_args;

/* Bytes of workspace csa2_sparse_attn needs for these arguments (may be 0). */
size_t csa2_attn_workspace_size(const csa2_attn_args* args);

int csa2_sparse_attn(const csa2_attn_args* args, void* ws, size_t ws_size, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H_ */
