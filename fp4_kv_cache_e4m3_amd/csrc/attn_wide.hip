// Sparse Top-K + sliding-window attention of one CSA2 layer for many query
// tokens at once (a prefill chunk), gfx950.
//
// Method: as in attn.hip (DeepSeek-V4.1-Flash pages, ai-maestro.online,
// "Compressed Sparse Attention 2" and "Causal Encoder-Decoder architecture";
// FP4 main KV per "FP4 KV, Bounded Replay, and other extensions"): the
// query's Top-K FP4 rows and its window rows share one softmax, one vector
// per entry is both key and value.
//
// Design.  With thousands of queries the work is a dense contraction per
// query (64 heads x 640 entries x 512 channels, twice), so this kernel is
// laid out for the matrix cores: one workgroup per (query, group of 64
// heads, head half hh of 32 heads), four waves (one per SIMD), 32-entry
// tiles.  Wave dq takes channel quarter dq (128 channels).  The two head
// halves of a query share nothing but their inputs, so they run as separate
// workgroups, two of which share a CU: their barriers are independent, and
// one workgroup's matrix work fills the SIMDs while the other waits at a
// barrier or in its softmax (with both halves in one workgroup, every
// barrier held all eight waves in the same phase).
//  * QK^T: wave dq contracts its channel quarter for the 32 heads (MFMA
//    16x16x32, entries as A rows, heads as B columns, Q in registers).  It
//    decodes only that quarter of the tile's FP4 rows, so a row is decoded
//    twice per query (once per head half).
//  * The four quarters' partial logits meet in LDS: wave dq adds the four
//    partials (in quarter order) of one 16 x 16 block, entries of subtile
//    dq / 2 and heads of tile dq % 2, and runs the online softmax on it; the
//    two waves holding a head's two entry halves exchange their tile
//    maxima, so both move the reference max together.  Every logit is
//    computed and exponentiated once.
//  * PV: wave dq owns output channels 128 dq .. + 127 of the 32 heads.  Those
//    are its own channel quarter, so it stages its own fp16 values in LDS
//    and reads them back transposed (ds_read_b64_tr_b16) as the B operand;
//    the probabilities of both head tiles come from LDS in the A-operand
//    layout of MFMA 16x16x32.
//  * Per tile: three barriers of four waves (partial logits, tile maxima,
//    probabilities).
// Precision as in attn.hip: FP4 values and bf16 Q are exact in fp16 (Q and
// window rows inside fp16's range); window logits run on bf16 MFMA with the
// bf16 Q; probabilities are fp16, normalised by the sum of the rounded values.
#include "attn_dev.h"

namespace csa2 {

namespace {
constexpr int kWD = 512;                // head dim
constexpr int kWTE = 32;                // entries per tile
constexpr int kWKQ = 4;                 // 32-channel k-steps per channel quarter
constexpr int kWVP = 128 + 8;           // halves per staged V row (the wave's channel quarter)
constexpr uint32_t kWOob = 0xFFFFF000u; // offset past every buffer
constexpr int kWDepth = 1;              // FP4 tiles in flight per wave

// FP4 data of two 16-entry subtiles for one lane: 32 channels (16 code bytes)
// and the scale word holding their two E4M3 scales, per entry
struct WRaw {
  uint32_t c[2][kWKQ];
  uint32_t s[2];
  bool v[2];                            // the entry exists
};

// window rows (bf16) of two 16-entry subtiles: 32 channels per entry
struct WRawW {
  u4 w[2][kWKQ];
};

CSA2_DEV v8bf half8_to_bf16(v8h x) {
  v8bf r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float)x[i];
  return r;
}
}  // namespace

template <bool PG>
__global__ __launch_bounds__(256, 2) void k_attn_wide(AttnParams p) {
  __shared__ __attribute__((aligned(16))) v4f xs[4][4 * 64];              // partial logits per wave
  __shared__ __attribute__((aligned(16))) _Float16 vst[4][kWTE * kWVP];   // staged V per wave
  __shared__ __attribute__((aligned(16))) v4h pg[2][2][64];               // probabilities [et][ht][lane]
  __shared__ float tmx[4][16];                                            // tile max per wave and head
  __shared__ float alph[32];                                              // rescale factor per head
  __shared__ int32_t rflag[2];                                            // per head tile: some head rescaled
  __shared__ float lsum[4][16];                                           // softmax sums per wave and head
  __shared__ int32_t spos[kMaxTopK];                                      // rows of the Top-K slots, -1 empty

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int dq = wave;
  const int et_o = dq >> 1, ht_o = dq & 1;          // the logit block this wave reduces
  const int partner = dq ^ 2;                       // the other entry half of the same heads
  const int cb = 128 * dq;                          // first output channel of the wave

  // workgroup -> (query, head group, head half): the two halves of a query
  // are neighbours, and consecutive queries share an XCD (the dispatcher
  // deals workgroup ids round-robin to the 8 XCDs), so a query's rows and
  // its neighbours' window rows share its L2
  const int ngr = (p.heads + 63) >> 6;
  const int64_t total = p.nq * ngr * 2;
  const int64_t per_xcd = (total + 7) >> 3;
  const int64_t uh = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (uh >= total) return;
  const int hh = (int)(uh & 1);
  const int64_t u = uh >> 1;
  const int q = (int)(u / ngr), grp = (int)(u - (int64_t)q * ngr);
  const int b = p.qn_shift >= 0 ? q >> p.qn_shift : q / p.qn;
  const int j = q - b * p.qn;
  const int h0 = 64 * grp;
  if (h0 + 32 * hh >= p.heads) return;             // a head half past H (H not a multiple of 64)

  // ---- Q: lane (n, g) holds, in k-step kk, channels 128 dq + 32 g + 8 kk ..
  // + 7 of head 32 hh + 16 ht + n (the k order inside an MFMA only has to
  // match the K rows')
  const rsrc_t q_buf = make_rsrc(p.q + ((int64_t)q * p.heads + h0) * kWD, (uint32_t)(min(64, p.heads - h0) * kWD * 2));
  u4 qraw[2][kWKQ];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int kk = 0; kk < kWKQ; ++kk) {
      const uint32_t off = 2u * (uint32_t)((32 * hh + 16 * ht + n) * kWD + 128 * dq + 32 * g + 8 * kk);
      qraw[ht][kk] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(q_buf, off, 0, 0));
    }

  // ---- Top-K slot s -> cache row (paged: through the block table), -1 empty
  const int nft = p.n_sparse_tiles > 0 ? (p.topk_k + kWTE - 1) / kWTE : 0;
  const int64_t row0 = PG ? 0 : (int64_t)b * p.T, nrows = PG ? p.cache_rows : p.T;
  const rsrc_t tk_buf = make_rsrc(p.topk + (int64_t)q * p.topk_k, (uint32_t)p.topk_k * 4u);
  const rsrc_t bt_buf = make_rsrc(PG ? p.block_table + (int64_t)b * p.max_pages : nullptr,
                                  PG ? (uint32_t)p.max_pages * 4u : 0u);
  auto slot_row = [&](int s) -> int32_t {
    const int32_t pos = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(tk_buf, s < p.topk_k ? 4u * (uint32_t)s : kWOob, 0, 0);
    int32_t row = s < p.topk_k && pos >= 0 && (int64_t)pos < p.T ? pos : -1;
    if constexpr (PG) {
      if (row >= 0) {
        const int32_t page = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(bt_buf, 4u * (uint32_t)(pos >> p.page_shift), 0, 0);
        const int64_t r = ((int64_t)page << p.page_shift) + (pos & ((1 << p.page_shift) - 1));
        row = page >= 0 && r < p.cache_rows ? (int32_t)r : -1;
      }
    }
    return row;
  };

  // ---- FP4 rows: lane (n, g) loads, for entry 32 i + 16 et + n, code bytes
  // 64 dq + 16 g .. + 15 and the aligned scale word holding scale bytes
  // 8 dq + 2 g, + 1
  const rsrc_t codes = make_rsrc(p.codes + row0 * p.codes_stride, (uint32_t)(nrows * p.codes_stride));
  const rsrc_t scales = make_rsrc(p.scales + row0 * p.scales_stride, (uint32_t)(nrows * p.scales_stride));
  const uint32_t lcb = (uint32_t)(64 * dq + 16 * g), lsb = (uint32_t)(8 * dq + 4 * (g >> 1));
  const uint32_t ssel = (uint32_t)(2 * (g & 1)) | (0x0Cu << 8) | ((uint32_t)(2 * (g & 1) + 1) << 16) | (0x0Cu << 24);
  auto load_rows = [&](const int32_t (&row)[2], WRaw& r) {
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      const uint32_t rc = row[et] >= 0 ? __umul24((uint32_t)row[et], (uint32_t)p.codes_stride) : kWOob;
      const uint32_t rs = row[et] >= 0 ? __umul24((uint32_t)row[et], (uint32_t)p.scales_stride) : kWOob;
      const u4 c = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(codes, rc + lcb, 0, 0));
      r.c[et][0] = c[0]; r.c[et][1] = c[1]; r.c[et][2] = c[2]; r.c[et][3] = c[3];
      r.s[et] = __builtin_amdgcn_raw_buffer_load_b32(scales, rs + lsb, 0, 0);
      r.v[et] = row[et] >= 0;
    }
  };
  // the first tiles' rows straight from the Top-K row, so their gathers go
  // out before anything waits; the other slots' rows go to LDS
  WRaw raw[kWDepth];
#pragma unroll
  for (int i = 0; i < kWDepth; ++i) {
    int32_t row[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) row[et] = i < nft ? slot_row(kWTE * i + 16 * et + n) : -1;
    load_rows(row, raw[i]);
  }
  for (int s = kWDepth * kWTE + threadIdx.x; s < nft * kWTE; s += 256) spos[s] = slot_row(s);
  v8h qf[2][kWKQ];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int kk = 0; kk < kWKQ; ++kk) qf[ht][kk] = bf16x8_to_half(qraw[ht][kk]);
  __syncthreads();                                  // spos
  auto load_fp4 = [&](int i, WRaw& r) {
    int32_t row[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) row[et] = i < nft ? spos[kWTE * i + 16 * et + n] : -1;
    load_rows(row, r);
  };

  // ---- window rows of window tile i: entry e = 32 i + 16 et + n is window
  // row j + e (ring slot (j + e + start) mod rows); lane (n, g) loads its 32
  // channels 128 dq + 32 g .. (64 bytes)
  const int first_swa = p.swa_len ? p.swa_rows - p.swa_len[b] : 0;
  int swa_st = p.swa_start ? p.swa_start[b] : 0;
  swa_st = swa_st >= 0 && swa_st < p.swa_rows ? swa_st : 0;
  const int nwt = (p.window + kWTE - 1) / kWTE;
  const rsrc_t swa_buf = make_rsrc(p.swa + (int64_t)b * p.swa_rows * kWD, (uint32_t)(p.swa_rows * kWD * 2));
  auto swa_valid = [&](int i, int et) {
    const int e = kWTE * i + 16 * et + n;
    const int r = j + e;
    return i < nwt && e < p.window && r >= first_swa && r < p.swa_rows;
  };
  auto load_swa = [&](int i, WRawW& r) {
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      const int e = kWTE * i + 16 * et + n;
      const int rr = j + e;
      const int rs = rr + swa_st >= p.swa_rows ? rr + swa_st - p.swa_rows : rr + swa_st;
      const uint32_t ro = swa_valid(i, et) ? (uint32_t)rs * (uint32_t)(2 * kWD) : kWOob;
#pragma unroll
      for (int kk = 0; kk < kWKQ; ++kk)
        r.w[et][kk] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 swa_buf, ro + 2u * (uint32_t)(128 * dq + 32 * g + 8 * kk), 0, 0));
    }
  };

  // O: o[a][t] holds heads 32 hh + 16 a + 4 g + i, channel cb + 16 t + n
  v4f o[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) o[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.0f;   // head 32 hh + 16 ht_o + n over entry half et_o

  _Float16* const my = &vst[wave][0];
  // V staging: lane (n, g) writes entry 16 et + n, channels 32 g + 8 kk of
  // the wave's quarter; transposing read: lane (n, g) gets entries
  // 16 et + 4 g .. + 3 of quarter channel 16 t + n
  _Float16* const vrow = my + n * kWVP + 32 * g;
  const _Float16* const vb = my + (4 * g + (n >> 2)) * kWVP + 4 * (n & 3);

  // the rest of a tile once the wave's partial logits acc[et][ht] (entries
  // 16 et + 4 g + i, head 32 hh + 16 ht + n, channel quarter dq) are in
  auto finish_tile = [&](v4f (&acc)[2][2], uint32_t vmask) {
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) xs[wave][(2 * et + ht) * 64 + lane] = acc[et][ht];
    __syncthreads();
    // logits of block (et_o, ht_o): the four quarters, added in quarter order
    v4f sfull = xs[0][dq * 64 + lane];
#pragma unroll
    for (int d = 1; d < 4; ++d) sfull += xs[d][dq * 64 + lane];
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool v = (vmask >> (16 * et_o + 4 * g + i)) & 1u;
      s[i] = v ? sfull[i] * p.qscale : -__builtin_inff();
    }
    float hmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    hmax = max_over_quarters(hmax);
    if (g == 0) tmx[wave][n] = hmax;
    __syncthreads();
    // online softmax of head n: both entry halves move the reference max
    // together (it moves only when the tile max exceeds it by more than 2^8,
    // so probabilities stay <= 256, fine for fp16)
    const float tmax = et_o == 0 ? fmaxf(hmax, tmx[partner][n]) : fmaxf(tmx[partner][n], hmax);
    const bool grow = tmax > m_run + 8.0f;
    const bool rs = grow && m_run != -__builtin_inff();
    const float alpha = rs ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;
    if (grow) m_run = tmax;
    const float mref = m_run == -__builtin_inff() ? 0.0f : m_run;
    v4h pr;
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = (_Float16)__builtin_amdgcn_exp2f(s[i] - mref);
    const v2h one2 = {(_Float16)1.0f, (_Float16)1.0f};
    const float ps = __builtin_amdgcn_fdot2(v2h{pr[2], pr[3]}, one2, __builtin_amdgcn_fdot2(v2h{pr[0], pr[1]}, one2, 0.0f, false), false);
    l_run = l_run * alpha + ps;
    pg[et_o][ht_o][lane] = pr;
    if (et_o == 0) {
      const bool any_rs = __any(rs);
      if (g == 0) alph[16 * ht_o + n] = alpha;
      if (lane == 0) rflag[ht_o] = any_rs ? 1 : 0;
    }
    __syncthreads();
    // rescale the O rows of every head tile that moved its max, then
    // O += P V over the 32 entries: k slot s of lane group g is entry
    // 4 g + s (s < 4) or 16 + 4 g + s - 4, in P and in V (two transposing
    // reads)
    v8h pa[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const v4h p0 = pg[0][a][lane];
      const v4h p1 = pg[1][a][lane];
      pa[a] = v8h{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      if (rflag[a]) {
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = alph[16 * a + 4 * g + i];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[a][t][i] *= ai[i];
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v4h v0 = lds_read_tr16(vb + 16 * t);
      const v4h v1 = lds_read_tr16(vb + 16 * kWVP + 16 * t);
      const v8h vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int a = 0; a < 2; ++a) o[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[a], vv, o[a][t], 0, 0, 0);
    }
  };

  auto tile_mask = [&](bool v0, bool v1) {
    return (uint32_t)(__ballot(v0) & 0xFFFFu) | ((uint32_t)(__ballot(v1) & 0xFFFFu) << 16);
  };

  // ---- FP4 tiles: kWDepth in flight; tile i + kWDepth is loaded into tile
  // i's registers as soon as tile i's logits are done with them
  if (nft > 0) {
    for (int i0 = 0; i0 < nft; i0 += kWDepth) {
#pragma unroll
      for (int uu = 0; uu < kWDepth; ++uu) {
        const int i = i0 + uu;
        if (i >= nft) break;
        const uint32_t vmask = tile_mask(raw[uu].v[0], raw[uu].v[1]);
        v4f acc[2][2] = {{v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}},
                         {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}};
        v2h sc[2];
#pragma unroll
        for (int et = 0; et < 2; ++et) sc[et] = e4m3_pair_s8(raw[uu].s[et], ssel);
#pragma unroll
        for (int kk = 0; kk < kWKQ; ++kk)
#pragma unroll
          for (int et = 0; et < 2; ++et) {
            const v8h kf = fp4x8_to_half_s8(raw[uu].c[et][kk], sc[et][kk >> 1]);
            acc[et][0] = mfma_qk(kf, qf[0][kk], acc[et][0]);
            acc[et][1] = mfma_qk(kf, qf[1][kk], acc[et][1]);
            *reinterpret_cast<v8h*>(vrow + 16 * et * kWVP + 8 * kk) = kf;
          }
        if (i + kWDepth < nft) load_fp4(i + kWDepth, raw[uu]);
        finish_tile(acc, vmask);
      }
    }
  }

  // ---- window tiles: bf16 logits against the bf16 Q (converted back from
  // the fp16 copy, exact for values that came from bf16); the next tile's
  // rows go out as soon as this tile's logits are done with its registers
  if (nwt > 0) {
    v8bf qb[2][kWKQ];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int kk = 0; kk < kWKQ; ++kk) qb[ht][kk] = half8_to_bf16(qf[ht][kk]);
    WRawW wr;
    load_swa(0, wr);
    for (int i = 0; i < nwt; ++i) {
      const uint32_t vmask = tile_mask(swa_valid(i, 0), swa_valid(i, 1));
      v4f acc[2][2] = {{v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}},
                       {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
      for (int kk = 0; kk < kWKQ; ++kk)
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          const v8bf kb = __builtin_bit_cast(v8bf, wr.w[et][kk]);
          acc[et][0] = mfma_qk(kb, qb[0][kk], acc[et][0]);
          acc[et][1] = mfma_qk(kb, qb[1][kk], acc[et][1]);
          *reinterpret_cast<v8h*>(vrow + 16 * et * kWVP + 8 * kk) = bf16x8_to_half(wr.w[et][kk]);
        }
      if (i + 1 < nwt) load_swa(i + 1, wr);
      finish_tile(acc, vmask);
    }
  }

  // ---- normalise: each head's sum over its two entry halves (in order)
  {
    float l = l_run + __shfl_xor(l_run, 16, 64);
    l = l + __shfl_xor(l, 32, 64);
    if (g == 0) lsum[wave][n] = l;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    // wave a owns head tile a's entry half 0, wave a + 2 its entry half 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = 32 * hh + 16 * a + 4 * g + i;  // head within the group
      const float l = lsum[a][4 * g + i] + lsum[a + 2][4 * g + i];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      if (h0 + hl < p.heads) {
        float* const orow = p.out + ((int64_t)q * p.heads + h0 + hl) * kWD + cb + n;
#pragma unroll
        for (int t = 0; t < 8; ++t) orow[16 * t] = o[a][t][i] * inv;
      }
    }
  }
}

hipError_t launch_attn_wide(const AttnParams& p, int nq, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  const int64_t total = (int64_t)nq * ((p.heads + 63) / 64) * 2;
  const dim3 grid((unsigned)(8 * ((total + 7) / 8)));
  if (p.block_table) hipLaunchKernelGGL(k_attn_wide<true>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_attn_wide<false>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace csa2
