// Internal definitions shared by the CSA2 gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

#define CSA2_DEV __device__ __forceinline__

namespace csa2 {

constexpr int kTopK = 512;
constexpr int kMaxTopK = 2048;                   // largest Top-K row the attention kernel takes
constexpr int kMaxSwaNew = 16;                   // largest Qn whose new 8-bit window rows the attention encodes
constexpr int kBlock = 8;
constexpr int kPoolBlocks = 2048;
constexpr int kPoolPositions = kPoolBlocks * kBlock;

// ---------------------------------------------------------------- ranking key
// Order-preserving map of an fp32 score to uint32: larger score -> larger key.
// -0.0 ranks with +0.0; every finite score maps to a key >= 1, so key 0 is
// free to mark "not a candidate".
CSA2_DEV uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- FP4 decode
// fp16 value of byte `sel` (a constant 0..3) of an E4M3FN word: the gfx950
// fp8 -> f32 convert decodes OCP E4M3FN exactly (0x7F / 0xFF -> NaN) and every
// finite E4M3 value is exact in fp16.
template <int SEL>
CSA2_DEV _Float16 e4m3_to_half(uint32_t word) {
  return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

// Eight E2M1 codes of one dword (channel 8w+i in nibble i, even channel in the
// low nibble of each byte) times one scale, as eight fp16 values in channel
// order.  The gfx950 FP4 -> fp16 convert applies only the power-of-two part of
// its fp32 scale operand, so it runs with scale 1.0 (exact E2M1 values) and
// one packed fp16 multiply applies the E4M3 scale.  E2M1 x E4M3 products have
// <= 6 significant bits and magnitudes in [2^-10, 2688], so every value and
// product is exact in fp16.
CSA2_DEV v8h fp4x8_to_half(uint32_t x, _Float16 s) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3);
  const v8h v = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  const v8h sv = {s, s, s, s, s, s, s, s};
  return v * sv;
}

// bf16 bits -> fp32 (exact)
CSA2_DEV float bf16_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// eight bf16 (two per dword) -> eight fp16, round to nearest even
CSA2_DEV v8h bf16x8_to_half(u4 w) {
  v8h r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
    r[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xFFFF0000u);
  }
  return r;
}

// ---------------------------------------------------------------- wave helpers
CSA2_DEV float wave_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// x + (x of lane l ^ 16), resp. l ^ 32, with the gfx950 permlane swaps (no LDS
// traffic); fp32 addition commutes, so both lanes get the same bits.
CSA2_DEV float sum_swap16(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
CSA2_DEV float sum_swap32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// ---------------------------------------------------------------- indexer dots
// Eight E4M3FN codes (byte i = element i) as eight fp16 values: the gfx950
// scaled fp8 -> fp16 convert with scale 1.0; every finite E4M3 value is exact
// in fp16.
CSA2_DEV v8h e4m3x8_to_half(uint32_t lo, uint32_t hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  const v8h v = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return v;
}

// One 16 x 16 tile of indexer dot products: score row 4g+i (A operand `a`)
// against token column n (B operand `b`) for lane (n, g), then ReLU.
// int8 operands: exact int32 dot products.  E4M3FN operands (F8): each
// 16-byte operand register is decoded to two groups of eight fp16 values
// (exact) that two fp16 MFMAs contract with fp32 accumulation; both operands
// are split alike, so every channel still meets its partner.  The products
// are exact, and the sums stay within the fp32 rounding model.  (The gfx950
// fp8 MFMA is not used here: its accumulation error, measured on random
// codes, reaches 2^-11 of the largest product.)
template <int KK, bool F8>
CSA2_DEV void index_dots(const v4i (&a)[KK], const v4i (&b)[KK], float (&d)[4]) {
  if constexpr (F8) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_half(a[kk][0], a[kk][1]),
                                                   e4m3x8_to_half(b[kk][0], b[kk][1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_half(a[kk][2], a[kk][3]),
                                                   e4m3x8_to_half(b[kk][2], b[kk][3]), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = fmaxf(acc[i], 0.0f);
  } else {
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[kk], b[kk], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = (float)max(acc[i], 0);
  }
}

}  // namespace csa2

// ---------------------------------------------------------------- launchers
namespace csa2 {

struct ScanParams {
  const int8_t* iq; const float* iw; const int8_t* ik; const int32_t* nvis;
  const float* iqs; const float* iks;                    // FP8 indexer: [nq, H_I] and [B, T] scales, else NULL
  int32_t batch, qn; int64_t T;
  uint32_t* tkeys; int64_t tk_stride;                    // [nq, tk_stride], or NULL: block maxima only
  uint32_t* bkeys; int64_t bk_stride;                    // [nq, bk_stride]
};
// FP4 quantisation of `rows` main-KV rows of `groups` 16-channel groups
// destination of new rows in a paged cache
struct PagedRows {
  const int32_t* seq; const int32_t* pos; const int32_t* bt;   // bt == NULL: contiguous rows
  int32_t batch, max_pages, shift; int64_t cache_rows;
};
struct QuantJob {
  const float* x; int64_t xs, rows; int32_t groups;
  uint8_t* codes; int64_t cs; uint8_t* scales; int64_t ss;
  PagedRows pg;                                          // pg.bt != NULL: rows go through a block table
};
struct SelectParams {
  const uint32_t* tkeys; int64_t tk_stride;
  const uint32_t* bkeys; int64_t bk_stride;
  const int32_t* nvis; int64_t T;
  int32_t* pool; int32_t* topk;                          // topk NULL: the pool only (> 8,192 blocks)
  int32_t roles;                                         // workgroups per query (set by the launcher)
  int32_t sel_wgs;                                       // selection workgroups (set by the launcher)
  QuantJob qj;                                           // rows == 0: none
  uint32_t* pkeys; uint32_t* pthr;                       // pool only: the pool blocks' keys [nq, 2048] and
                                                         // the Top-512 key floor [nq], or NULL
};
struct ReindexParams {
  const int8_t* iq; const float* iw; const int8_t* ik; const int32_t* nvis;
  const float* iqs; const float* iks;                    // FP8 indexer scales, else NULL
  const int32_t* pool; int32_t qn; int64_t T;
  uint32_t* ckeys;                                       // [nq, 16384]
  int32_t* topk;
  uint32_t* bkeys;                                       // [nq, 2048]: max key of each pool block
  const uint32_t* pkeys; const uint32_t* pthr;           // or NULL: pool blocks whose key is below the
                                                         // floor are not rescored (long Full path)
};
struct AttnParams {
  const uint16_t* q; const uint8_t* codes; const uint8_t* scales;
  const int32_t* topk; const uint16_t* swa; const int32_t* swa_len;
  float* out; float* opart; float* mlpart;
  int64_t T, codes_stride, scales_stride, nq;
  int32_t qn, heads, topk_k, window, swa_rows, splits, tiles_per_split, n_sparse_tiles, n_tiles;
  int32_t qn_shift;                                      // log2(qn) when qn is a power of two, else -1
  float qscale;                                          // sm_scale * log2(e)
  int32_t swa_fp8;                                       // window rows: 0 bf16, 1 E4M3 codes + row scales
  const float* swa_scale;                                // [B, swa_rows] powers of two (swa_fp8)
  const int32_t* block_table;                            // paged cache [B, max_pages], or NULL
  int32_t max_pages, page_shift;
  int64_t cache_rows;                                    // physical rows of a paged cache
  const int32_t* swa_start;                              // ring slot of window row 0 per sequence, or NULL
  const uint16_t* swa_new;                               // S8: the step's new window rows (bf16 [B * Qn, d]), or NULL
  int32_t* rows_out;                                     // paged: the Top-K slots' cache rows [nq, topk_k], or NULL
  int32_t rows_in;                                       // 1: topk holds cache rows (no block table)
};

hipError_t launch_quantize(const float* x, int64_t xs, int64_t rows, int dim, uint8_t* codes,
                           int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st);
hipError_t launch_quantize_paged(const float* x, int64_t xs, int64_t rows, int dim, const PagedRows& d,
                                 uint8_t* codes, int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st);
bool quantize_fits_quad(int64_t rows, int dim);           // small enough for four lanes per group
hipError_t launch_quantize_swa8(const uint16_t* x, int64_t xs, int64_t rows, int dim, uint8_t* out, int64_t os,
                                float* scales, int64_t ss, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, int64_t cs, const uint8_t* scales, int64_t ss,
                             int64_t rows, int dim, float* out, int64_t os, hipStream_t st);
hipError_t launch_index_scan(const ScanParams& p, int heads, int dim, hipStream_t st);
hipError_t launch_select_full(const SelectParams& p, int nq, int64_t max_blocks, hipStream_t st);
hipError_t launch_reindex(const ReindexParams& p, int nq, int heads, int dim, hipStream_t st);
hipError_t launch_attn(const AttnParams& p, int nq, int dim, int waves, hipStream_t st);
hipError_t launch_attn_wide(const AttnParams& p, int nq, hipStream_t st);   // dim 512, bf16 window

}  // namespace csa2
