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
// heads), four waves, 32-entry tiles.  Wave w = (hh, dh): head half hh (32
// heads), channel half dh (256 channels).
//  * QK^T: wave (hh, dh) contracts its channel half for its 32 heads
//    (MFMA 16x16x32, entries as A rows, heads as B columns; Q is read from
//    LDS, lane-contiguous, once per k-step).  Each wave decodes only its own channel half of the tile's
//    FP4 rows, so a row is decoded twice per workgroup (once per head half),
//    not once per head group.  The two channel halves' partial logits meet
//    through LDS and are added in a fixed order, so both waves of a head half
//    hold bit-identical logits and run the same online softmax.
//  * PV: wave (hh, dh) owns output channel quarter 2 dh + hh for all 64
//    heads (O in 128 accumulator registers).  That quarter lies inside the
//    channel half the wave decoded, so it stages its own fp16 values in LDS
//    and reads them back transposed (ds_read_b64_tr_b16) as the B operand;
//    the probabilities of its own head half are already in the A-operand
//    layout of MFMA 16x16x32, those of the other half come through LDS (with
//    their rescale factors).
//  * Per tile: two barriers (partial logits, probabilities).
// Precision as in attn.hip: FP4 values and bf16 Q are exact in fp16 (Q and
// window rows inside fp16's range); window logits run on bf16 MFMA with the
// bf16 Q; probabilities are fp16, normalised by the sum of the rounded values.
#include "attn_dev.h"

namespace csa2 {

namespace {
constexpr int kWD = 512;                // head dim
constexpr int kWTE = 32;                // entries per tile
constexpr int kWKH = 8;                 // 32-channel k-steps per channel half
constexpr int kWVP = 128 + 8;           // halves per staged V row (one channel quarter)
constexpr uint32_t kWOob = 0xFFFFF000u; // offset past every buffer

// FP4 data of two 16-entry subtiles for one lane: 64 channels (32 code bytes)
// and their four E4M3 scales per entry
struct WRaw {
  uint32_t c[2][kWKH];
  uint32_t s[2];
  bool v[2];                            // the entry exists
};

// window rows (bf16) of two 16-entry subtiles: 64 channels per entry
struct WRawW {
  u4 w[2][kWKH];
};

CSA2_DEV v8bf half8_to_bf16(v8h x) {
  v8bf r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)(float)x[i];
  return r;
}
}  // namespace

template <bool PG>
__global__ __launch_bounds__(256, 1) void k_attn_wide(AttnParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 vst[4][kWTE * kWVP];   // staged V per wave
  __shared__ __attribute__((aligned(16))) v4f xs[4][4 * 64];              // partial logits per wave
  __shared__ __attribute__((aligned(16))) v8h pbuf[2][2 * 64];            // probabilities per head half
  __shared__ float alph[2][32];                                           // rescale factors per head half
  __shared__ float lsum[2][32];                                           // softmax sums per head half
  __shared__ int32_t rflag[2];
  __shared__ int32_t spos[kMaxTopK];                                      // rows of the Top-K slots, -1 empty
  __shared__ __attribute__((aligned(16))) u4 qlds[4][2 * kWKH * 64];      // each wave's Q operands

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int hh = wave & 1, dh = wave >> 1, cq = 2 * dh + hh;
  const bool stager = (g >> 1) == hh;     // this lane's 64 channels lie in the wave's output quarter

  // workgroup -> (query, head group): consecutive queries on one XCD (the
  // dispatcher deals workgroup ids round-robin to the 8 XCDs), so a query's
  // neighbours, which share most of its window rows, share its L2
  const int ngr = (p.heads + 63) >> 6;
  const int64_t total = p.nq * ngr;
  const int64_t per_xcd = (total + 7) >> 3;
  const int64_t u = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= total) return;
  const int q = (int)(u / ngr), grp = (int)(u - (int64_t)q * ngr);
  const int b = p.qn_shift >= 0 ? q >> p.qn_shift : q / p.qn;
  const int j = q - b * p.qn;
  const int h0 = 64 * grp;

  // ---- Q: this wave's 32 heads x 256 channels as the QK^T B operand; lane
  // (n, g) holds, in k-step kk, channels 256 dh + 64 g + 8 kk .. + 7 of head
  // 32 hh + 16 ht + n (the k order inside an MFMA only has to match the K
  // rows').  Kept in LDS (fp16; bf16 for the window tiles), one 16-byte
  // operand per lane and (ht, kk), wave-private, read back lane-contiguous.
  // The loads go out first; they are converted once the first gathers are out.
  const rsrc_t q_buf = make_rsrc(p.q + ((int64_t)q * p.heads + h0) * kWD, (uint32_t)(min(64, p.heads - h0) * kWD * 2));
  u4* const myq = &qlds[wave][0];
  u4 qraw[2 * kWKH];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int kk = 0; kk < kWKH; ++kk) {
      const uint32_t off = 2u * (uint32_t)((32 * hh + 16 * ht + n) * kWD + 256 * dh + 64 * g + 8 * kk);
      qraw[ht * kWKH + kk] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(q_buf, off, 0, 0));
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

  // ---- FP4 rows of tile i: lane (n, g) loads, for entry 32 i + 16 et + n,
  // code bytes 128 dh + 32 g .. + 31 and scale bytes 16 dh + 4 g .. + 3
  const rsrc_t codes = make_rsrc(p.codes + row0 * p.codes_stride, (uint32_t)(nrows * p.codes_stride));
  const rsrc_t scales = make_rsrc(p.scales + row0 * p.scales_stride, (uint32_t)(nrows * p.scales_stride));
  const uint32_t lcb = (uint32_t)(128 * dh + 32 * g), lsb = (uint32_t)(16 * dh + 4 * g);
  auto load_rows = [&](const int32_t (&row)[2], WRaw& r) {
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      const uint32_t rc = row[et] >= 0 ? __umul24((uint32_t)row[et], (uint32_t)p.codes_stride) : kWOob;
      const uint32_t rs = row[et] >= 0 ? __umul24((uint32_t)row[et], (uint32_t)p.scales_stride) : kWOob;
      const u4 c0 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(codes, rc + lcb, 0, 0));
      const u4 c1 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(codes, rc + lcb + 16, 0, 0));
      r.c[et][0] = c0[0]; r.c[et][1] = c0[1]; r.c[et][2] = c0[2]; r.c[et][3] = c0[3];
      r.c[et][4] = c1[0]; r.c[et][5] = c1[1]; r.c[et][6] = c1[2]; r.c[et][7] = c1[3];
      r.s[et] = __builtin_amdgcn_raw_buffer_load_b32(scales, rs + lsb, 0, 0);
      r.v[et] = row[et] >= 0;
    }
  };
  // the first two tiles' rows straight from the Top-K row, so their gathers
  // go out before anything waits; the other slots' rows go to LDS
  WRaw raw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int32_t row[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) row[et] = i < nft ? slot_row(kWTE * i + 16 * et + n) : -1;
    load_rows(row, raw[i]);
  }
  for (int s = 2 * kWTE + threadIdx.x; s < nft * kWTE; s += 256) spos[s] = slot_row(s);
#pragma unroll
  for (int f = 0; f < 2 * kWKH; ++f) myq[f * 64 + lane] = __builtin_bit_cast(u4, bf16x8_to_half(qraw[f]));
  __syncthreads();                                  // spos
  auto load_fp4 = [&](int i, WRaw& r) {
    int32_t row[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) row[et] = i < nft ? spos[kWTE * i + 16 * et + n] : -1;
    load_rows(row, r);
  };

  // ---- window rows of window tile i: entry e = 32 i + 16 et + n is window
  // row j + e (ring slot (j + e + start) mod rows); lane (n, g) loads its 64
  // channels 256 dh + 64 g .. (128 bytes)
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
      for (int kk = 0; kk < kWKH; ++kk)
        r.w[et][kk] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 swa_buf, ro + 2u * (uint32_t)(256 * dh + 64 * g + 8 * kk), 0, 0));
    }
  };

  // O rows of the wave's own head half (oo) and of the other one (ox):
  // oo[ht][t] holds heads 32 hh + 16 ht + 4 g + i, ox those of half hh ^ 1,
  // channel 128 cq + 16 t + n (static indices only: the arrays stay in
  // registers)
  v4f oo[2][8], ox[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      oo[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
      ox[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.0f, 0.0f};

  _Float16* const my = &vst[wave][0];
  // V staging: lane (n, g) (stager) writes entry 16 et + n, quarter channels
  // 64 (g & 1) + 8 kk; transposing read: lane (n, g) gets entries
  // 16 et + 4 g .. + 3 of quarter channel 16 t + n
  _Float16* const vrow = my + n * kWVP + 64 * (g & 1);
  const _Float16* const vb = my + (4 * g + (n >> 2)) * kWVP + 4 * (n & 3);

  // the rest of a tile once the wave's partial logits acc[et][ht] (entries
  // 16 et + 4 g + i, head 32 hh + 16 ht + n, channel half dh) are in
  auto finish_tile = [&](v4f (&acc)[2][2], uint32_t vmask) {
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) xs[wave][(2 * et + ht) * 64 + lane] = acc[et][ht];
    __syncthreads();
    // logits: channel half 0 + channel half 1, in that order in both waves
    float s[2][2][4];
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const v4f other = xs[wave ^ 2][(2 * et + ht) * 64 + lane];
        const v4f full = dh == 0 ? acc[et][ht] + other : other + acc[et][ht];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = (vmask >> (16 * et + 4 * g + i)) & 1u;
          s[et][ht][i] = v ? full[i] * p.qscale : -__builtin_inff();
        }
      }
    // online softmax per head (lane n, head half ht); the reference max moves
    // only when a tile's max exceeds it by more than 2^8 (probabilities stay
    // <= 256, fine for fp16)
    v8h pr[2];
    float alpha[2];
    bool resc = false;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float tmax = -__builtin_inff();
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[et][ht][i]);
      tmax = max_over_quarters(tmax);
      const bool grow = tmax > m_run[ht] + 8.0f;
      const bool rs = grow && m_run[ht] != -__builtin_inff();
      alpha[ht] = rs ? __builtin_amdgcn_exp2f(m_run[ht] - tmax) : 1.0f;
      resc |= rs;
      if (grow) m_run[ht] = tmax;
      const float mref = m_run[ht] == -__builtin_inff() ? 0.0f : m_run[ht];
#pragma unroll
      for (int et = 0; et < 2; ++et)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[ht][4 * et + i] = (_Float16)__builtin_amdgcn_exp2f(s[et][ht][i] - mref);
      const v2h one2 = {(_Float16)1.0f, (_Float16)1.0f};
      float ps = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) ps = __builtin_amdgcn_fdot2(v2h{pr[ht][2 * k], pr[ht][2 * k + 1]}, one2, ps, false);
      l_run[ht] = l_run[ht] * alpha[ht] + ps;
    }
    const bool any_resc = __any(resc);
    if (dh == 0) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        pbuf[hh][ht * 64 + lane] = pr[ht];
        if (g == 0) alph[hh][16 * ht + n] = alpha[ht];
      }
      if (lane == 0) rflag[hh] = any_resc ? 1 : 0;
    }
    __syncthreads();
    v8h po[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) po[ht] = pbuf[hh ^ 1][ht * 64 + lane];
    // rescale O rows (heads 16 a + 4 g + i) of either half that moved its max
    if (any_resc) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha[ht], 4 * g + i, 64);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) oo[ht][t][i] *= ai[i];
      }
    }
    if (rflag[hh ^ 1]) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = alph[hh ^ 1][16 * ht + 4 * g + i];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) ox[ht][t][i] *= ai[i];
      }
    }
    // O += P V over the 32 entries: k slot s of lane group g is entry
    // 4 g + s (s < 4) or 16 + 4 g + s - 4, in P (from the logits' layout) and
    // in V (two transposing reads)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v4h v0 = lds_read_tr16(vb + 16 * t);
      const v4h v1 = lds_read_tr16(vb + 16 * kWVP + 16 * t);
      const v8h vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        oo[ht][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr[ht], vv, oo[ht][t], 0, 0, 0);
        ox[ht][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(po[ht], vv, ox[ht][t], 0, 0, 0);
      }
    }
  };

  auto tile_mask = [&](bool v0, bool v1) {
    return (uint32_t)(__ballot(v0) & 0xFFFFu) | ((uint32_t)(__ballot(v1) & 0xFFFFu) << 16);
  };

  // ---- FP4 tiles: two in flight; tile i + 2 is loaded into tile i's
  // registers as soon as tile i's logits are done with them
  if (nft > 0) {
    for (int i0 = 0; i0 < nft; i0 += 2) {
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int i = i0 + uu;
        if (i >= nft) break;
        const uint32_t vmask = tile_mask(raw[uu].v[0], raw[uu].v[1]);
        v4f acc[2][2] = {{v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}},
                         {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}};
        v2h sa[2], sb[2];
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          sa[et] = e4m3_pair_s8(raw[uu].s[et], 0x0C010C00u);
          sb[et] = e4m3_pair_s8(raw[uu].s[et], 0x0C030C02u);
        }
#pragma unroll
        for (int kk = 0; kk < kWKH; ++kk) {
          const v8h q0 = __builtin_bit_cast(v8h, myq[kk * 64 + lane]);
          const v8h q1 = __builtin_bit_cast(v8h, myq[(kWKH + kk) * 64 + lane]);
#pragma unroll
          for (int et = 0; et < 2; ++et) {
            const _Float16 s8 = kk < 4 ? sa[et][kk >> 1] : sb[et][(kk >> 1) - 2];
            const v8h kf = fp4x8_to_half_s8(raw[uu].c[et][kk], s8);
            acc[et][0] = mfma_qk(kf, q0, acc[et][0]);
            acc[et][1] = mfma_qk(kf, q1, acc[et][1]);
            if (stager) *reinterpret_cast<v8h*>(vrow + 16 * et * kWVP + 8 * kk) = kf;
          }
        }
        if (i + 2 < nft) load_fp4(i + 2, raw[uu]);
        finish_tile(acc, vmask);
      }
    }
  }

  // ---- window tiles: bf16 logits against the bf16 Q (converted back from
  // the fp16 copy, exact for values that came from bf16); the next tile's
  // rows are loaded as soon as this tile's logits are done
  if (nwt > 0) {
#pragma unroll
    for (int f = 0; f < 2 * kWKH; ++f)
      myq[f * 64 + lane] = __builtin_bit_cast(u4, half8_to_bf16(__builtin_bit_cast(v8h, myq[f * 64 + lane])));
    WRawW wr;
    load_swa(0, wr);
    for (int i = 0; i < nwt; ++i) {
      const uint32_t vmask = tile_mask(swa_valid(i, 0), swa_valid(i, 1));
      v4f acc[2][2] = {{v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}},
                       {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
      for (int kk = 0; kk < kWKH; ++kk) {
        const v8bf q0 = __builtin_bit_cast(v8bf, myq[kk * 64 + lane]);
        const v8bf q1 = __builtin_bit_cast(v8bf, myq[(kWKH + kk) * 64 + lane]);
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          const v8bf kb = __builtin_bit_cast(v8bf, wr.w[et][kk]);
          acc[et][0] = mfma_qk(kb, q0, acc[et][0]);
          acc[et][1] = mfma_qk(kb, q1, acc[et][1]);
          if (stager) *reinterpret_cast<v8h*>(vrow + 16 * et * kWVP + 8 * kk) = bf16x8_to_half(wr.w[et][kk]);
        }
      }
      if (i + 1 < nwt) load_swa(i + 1, wr);
      finish_tile(acc, vmask);
    }
  }

  // ---- normalise: the sums of every head of both halves
  float lt[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    float l = l_run[ht] + __shfl_xor(l_run[ht], 16, 64);
    lt[ht] = l + __shfl_xor(l, 32, 64);
  }
  if (dh == 0 && g == 0) {
    lsum[hh][n] = lt[0];
    lsum[hh][16 + n] = lt[1];
  }
  __syncthreads();
  auto store_half = [&](const v4f (&oh)[2][8], int half) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hl = 32 * half + 16 * ht + 4 * g + i;  // head within the group
        const float l = lsum[half][16 * ht + 4 * g + i];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        if (h0 + hl < p.heads) {
          float* const orow = p.out + ((int64_t)q * p.heads + h0 + hl) * kWD + 128 * cq + n;
#pragma unroll
          for (int t = 0; t < 8; ++t) orow[16 * t] = oh[ht][t][i] * inv;
        }
      }
  };
  store_half(oo, hh);
  store_half(ox, hh ^ 1);
}

hipError_t launch_attn_wide(const AttnParams& p, int nq, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  const int64_t total = (int64_t)nq * ((p.heads + 63) / 64);
  const dim3 grid((unsigned)(8 * ((total + 7) / 8)));
  if (p.block_table) hipLaunchKernelGGL(k_attn_wide<true>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_attn_wide<false>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace csa2
