// Sparse Top-K + sliding-window attention of one CSA2 layer for gfx950.
//
// Method: DeepSeek-V4.1-Flash pages.  Each layer keeps its own main Q and its
// own sliding-window cache and attends over the Top-K entries its Full /
// Reindex layer selected (Reuse layers take the latest ones):
// ai-maestro.online, "Compressed Sparse Attention 2"; the window is 128 tokens
// ("Causal Encoder-Decoder architecture"); the main KV is FP4 E2M1 with one
// E4M3 scale per 16 channels ("FP4 KV, Bounded Replay, and other
// extensions").  The sparse entries and the window rows share one softmax
// (merged by an online softmax over 16-entry tiles); one vector per entry is
// both key and value.
//
// Work decomposition (wave64, MFMA):
//  * workgroup = (query, group of 16 heads, split of the tile list, column
//    half of the output channels).  Both halves of a (query, head group)
//    compute the same logits over all D channels; each stages and multiplies
//    only its own D/2 value channels, so no partial outputs are exchanged.
//    All workgroups of one query get ids that are equal mod 8, which the
//    dispatcher places on one XCD, so they share its L2 for the query's rows.
//  * NW waves per workgroup take every NW-th 16-entry tile and merge their
//    (max, sum, O) states through LDS at the end; when the tile list is split
//    over several workgroups, a second kernel merges the partial states.
//  * per tile a wave gathers 16 entries (lane % 16 = entry; the 4 lanes of an
//    entry split its channels) through buffer loads, FP4 codes + E4M3 scales
//    or bf16 window rows.  Every load is unconditional (absent data reads
//    zeros through out-of-range offsets), so the compiler's wait counts are
//    exact and two FP4 gathers stay in flight per wave; the last FP4 pair
//    loads the wave's first window tile instead.
//  * QK^T: MFMA 16x16x32 with the entries as A rows and the 16 heads as B
//    columns.  FP4 rows become fp16 in registers (exact) against an fp16
//    copy of Q; window rows stay bf16 against a bf16 copy of Q.  The own
//    half of Q lives in registers, the other half is read from LDS per
//    k-step.  Each half's k-steps accumulate separately and the two sums are
//    added last; fp32 addition commutes, so both column halves get
//    bit-identical logits whichever half they process first.  The result
//    holds entries 4*(lane/16)+i of head lane%16 -- the A-operand layout of
//    the PV MFMA, so the probabilities never leave registers.
//  * PV: MFMA 16x16x16 f16 over the 16 entries; the V operand (4 entries of
//    one channel per lane) comes from one transposing LDS read per 16
//    channels of the wave's own fp16 half-tile.
// Q goes bf16 -> fp16 unscaled for the FP4 tiles, which is exact for
// magnitudes in [2^-14, 65504] (bf16 carries 8 significant bits, fp16 11);
// products are exact in both MFMA types, so QK^T is exact up to fp32
// accumulation.  sm_scale * log2(e) multiplies the fp32 logits and the
// softmax uses exp2.
#include "attn_dev.h"
#include "quant_dev.h"

namespace csa2 {

// Geometry of one lane's share of a 16-entry tile for head dim D.
template <int D>
struct Geo {
  static constexpr int HALF = D / 2;       // channels per column half
  static constexpr int CPL = D / 8;        // channels per lane per half
  static constexpr int KH = CPL / 8;       // 32-channel k-steps per half (8 channels per lane each)
  static constexpr int NT = HALF / 16;     // 16-channel PV tiles per half
  static constexpr int PITCH = HALF + 8;   // LDS row pitch of a half-tile, in halves
};

// Column halves.  Each workgroup owns one half of the output channels.  The
// halves interleave in blocks: the D channels form 4 blocks of BLK = D/4, and
// half ch holds the second half of every block if ch = 1, the first if ch = 0.
// A half's channels are numbered o = 0 .. D/2-1 ("half index"); gch(o, ch) is
// the channel of half index o.  This way lane g of an FP4 entry owns block g
// outright -- both its halves, BLK/2 contiguous code bytes and BLK/16
// contiguous scale bytes -- so a tile's gather is one wide load per 16 code
// bytes and a single load for the scales.
template <int D>
struct Halves {
  static constexpr int BLK = D / 4;
  static constexpr int SUB = BLK / 2;                 // channels of a half in one block
  static constexpr int gch(int o, int ch) { return BLK * (o / SUB) + SUB * ch + (o % SUB); }
};

// Lane -> half-index maps (a lane holds 8 channels per 32-channel k-step j;
// lanes g = 0..3 of an entry share the k-step).  The QK contraction does not
// care about the channel order as long as K and Q use the same map, so each
// data type gets the map that suits its loads; off(j) + LANE * g is the half
// index of the lane's first channel of k-step j.
//  * FP4 codes ("blocks"): lane g holds half indices SUB*g .. SUB*g + SUB - 1,
//    i.e. its own block.
//  * bf16 window rows ("interleaved"): k-step j, lane g holds half indices
//    32j + 8g .. +7; the 4 lanes of a row read contiguous bytes.
template <int D>
struct BlockMap {
  static constexpr int LANE = Halves<D>::SUB;
  static constexpr int off(int j) { return 8 * j; }
};
template <int D>
struct InterMap {
  static constexpr int LANE = 8;
  static constexpr int off(int j) { return 32 * j; }
};

// 8-bit window rows ("pairs"): k-steps 2i and 2i+1 of lane g hold the 16
// consecutive half indices 64i + 16g .. +15, so one 16-byte load covers two
// k-steps.
template <int D>
struct Fp8Map {
  static constexpr int LANE = 16;
  static constexpr int off(int j) { return 64 * (j / 2) + 8 * (j % 2); }
};

// Eight E4M3 window codes (two dwords, channel order) times the row's
// power-of-two scale, as fp16: the gfx950 scaled FP8 -> fp16 conversion
// applies the power of two itself; E4M3 values times 2^k are exact in fp16
// for k in [-15, 7] (row maxima from about 0.014 to 57,344).
CSA2_DEV v8h fp8x8_to_half(uint32_t w0, uint32_t w1, float sc) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, sc, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, sc, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, sc, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, sc, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// FP4 data of one entry for this lane (BlockMap): code words w[h][j] of
// k-step j of half h (h = 0: the workgroup's own half) and the scale bytes of
// the lane's block as loaded (D = 512: s[0] = groups 8g .. 8g+3, s[1] =
// groups 8g+4 .. 8g+7; D = 128: one word holding groups 2g, 2g+1).  The
// scale bytes are picked out where they are used, so issuing a gather never
// waits for its own data.
template <int D>
struct Fp4Raw {
  uint32_t w[2][Geo<D>::KH];
  uint32_t s[2];
};

// One sequence's FP4 rows as buffers, plus this lane's fixed offsets.  A row
// offset at or past `oob` lies outside both buffers, so an empty Top-K slot
// reads zero codes and zero scales.
struct Fp4Src {
  rsrc_t codes, scales;
  uint32_t cstride, sstride, oob;
  int hcb[2];                  // code byte offset of each half within the lane's block (0 = own)
  uint32_t lcb, lsb;           // per-lane code / scale byte offset (the lane's block)
};

template <int D>
CSA2_DEV bool load_fp4(const Fp4Src& src, int32_t pos, uint32_t T, Fp4Raw<D>& r) {
  using G = Geo<D>;
  const bool valid = pos >= 0 && (uint32_t)pos < T;
  const uint32_t rc = valid ? __umul24((uint32_t)pos, src.cstride) : src.oob;
  const uint32_t rs = valid ? __umul24((uint32_t)pos, src.sstride) : src.oob;
  // the loads go out in one fixed order wherever a gather is issued, so the
  // compiler's count of loads in flight is the same on every path into a tile
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (G::KH == 8) {
      // a half of the lane's block: 32 code bytes, two 16-byte loads
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u4 c = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                src.codes, rc + src.lcb + 16 * i, src.hcb[h], 0));
        r.w[h][4 * i + 0] = c[0]; r.w[h][4 * i + 1] = c[1];
        r.w[h][4 * i + 2] = c[2]; r.w[h][4 * i + 3] = c[3];
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      static_assert(G::KH == 2, "D must be 128 or 512");
      const u2 c = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(src.codes, rc + src.lcb, src.hcb[h], 0));
      r.w[h][0] = c[0]; r.w[h][1] = c[1];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (G::KH == 8) {
    const u2 s = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(src.scales, rs + src.lsb, 0, 0));
    r.s[0] = s[0]; r.s[1] = s[1];
  } else {
    r.s[0] = __builtin_amdgcn_raw_buffer_load_b32(src.scales, rs + src.lsb, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  return valid;
}


// One 16-entry tile: logits, online-softmax update, O += P V for the own half.
// kvf(h, j) gives this lane's 8 channels of k-step j of half h under channel
// map M as a QK operand of type V8 (fp16 for FP4 rows, the raw bf16 for window
// rows); qop(h, j) gives the matching Q channels (the own half from
// registers, the other half from registers or LDS).  stage(kv) turns an
// own-half operand into the
// fp16 V values staged at wrow (this lane's LDS row plus M::LANE * g) for PV;
// after_qk() runs once the raw tile data has been consumed.
template <int D, typename M, typename V8, typename KV, typename QO, typename ST, typename AfterQK>
CSA2_DEV void attend_tile(const AttnParams& p, KV kvf, QO qop, ST stage, AfterQK after_qk, bool valid,
                          _Float16* wrow, const _Float16* vbase, int g, v4f (&o)[Geo<D>::NT], float& m_run,
                          float& l_run) {
  constexpr int KH = Geo<D>::KH, NT = Geo<D>::NT;
  // one accumulation chain per half (the two halves interleave); the half sums
  // are added last
  v4f part[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < KH; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const V8 kv = kvf(h, j);
      const V8 qv = qop(h, j);
      part[h] = mfma_qk(kv, qv, part[h]);
      if (h == 0) *reinterpret_cast<v8h*>(wrow + M::off(j)) = stage(kv);
    }
  }
  const v4f s_acc = part[0] + part[1];      // commutative: same bits in both halves
  after_qk();                               // the tile's raw data is dead from here on

  // online softmax (head = lane % 16, entries 4g..4g+3).  The reference max
  // only moves when a tile's max exceeds it by more than 2^8, so O is rarely
  // rescaled; probabilities stay <= 256, fine for fp16.  Masked entries get
  // -inf logits (probability exactly 0).
  const uint64_t vm = __ballot(valid);
  float s4[4];
  if (vm == ~0ull) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = s_acc[i] * p.qscale;
  } else {
    const uint32_t bits = (uint32_t)(vm >> (4 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = ((bits >> i) & 1u) ? s_acc[i] * p.qscale : -__builtin_inff();
  }
  float tmax = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
  tmax = max_over_quarters(tmax);
  const bool grow = tmax > m_run + 8.0f;
  // a wave's first entries only set the reference (O and l are still zero)
  const bool rescale = grow && m_run != -__builtin_inff();
  float alpha = 1.0f;
  if (rescale) alpha = __builtin_amdgcn_exp2f(m_run - tmax);
  if (grow) m_run = tmax;
  const float mref = m_run == -__builtin_inff() ? 0.0f : m_run;   // all masked so far: exp2(-inf) = 0
  v4h pa;
#pragma unroll
  for (int i = 0; i < 4; ++i) pa[i] = (_Float16)__builtin_amdgcn_exp2f(s4[i] - mref);
  // normalise with the probabilities actually used (fp16 products with 1 are exact)
  const v2h one2 = {(_Float16)1.0f, (_Float16)1.0f};
  const float psum = __builtin_amdgcn_fdot2(v2h{pa[2], pa[3]}, one2, __builtin_amdgcn_fdot2(v2h{pa[0], pa[1]}, one2, 0.0f, false), false);
  l_run = l_run * alpha + psum;
  if (__any(rescale)) {
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t][i] *= ai[i];
  }

  // O += P V: the V operand (4 entries of one channel per lane) comes from one
  // transposing LDS read per 16-channel tile
  wave_lds_sync();
#pragma unroll
  for (int t = 0; t < NT; ++t)
    o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, lds_read_tr16(vbase + 16 * t), o[t], 0, 0, 0);
  wave_lds_sync();
}

// S8: the window rows are 8-bit (E4M3 codes + a power-of-two scale per row)
// instead of bf16; with p.swa_new the step's new rows arrive as bf16, are
// encoded by every workgroup of the sequence into LDS (read from there, not
// from the cache) and stored into the cache by one workgroup of the sequence.
// PG: 0 contiguous cache ([B, T] rows), 1 paged cache (Top-K positions go
// through the block table; with p.rows_out one workgroup per query and
// split also writes the rows it found), 2 the Top-K row already holds cache
// rows (a paged call's rows_out)
template <int D, int NW, bool S8, int PG>
__global__ __launch_bounds__(64 * NW, 2) void k_attn(AttnParams p) {
  using G = Geo<D>;
  constexpr int KH = G::KH, NT = G::NT, PITCH = G::PITCH, HALF = G::HALF;
  constexpr int TILE_HALVES = 16 * PITCH;
  constexpr int QPITCH = D + 8;
  // one LDS arena: per-wave V half-tiles, Q of the 16 heads and this split's
  // Top-K positions while the tiles run; the NW partial outputs at the merge
  constexpr int VT_BYTES = NW * TILE_HALVES * 2, QS_BYTES = 16 * QPITCH * 2, SPOS_BYTES = kMaxTopK * 4;
  // S8: the step's new window rows, encoded by the workgroup itself (codes
  // [kMaxSwaNew][D], then their row scales)
  constexpr int NEW_BYTES = S8 ? kMaxSwaNew * (D + 4) : 0;
  constexpr int WORK_BYTES = VT_BYTES + 2 * QS_BYTES + SPOS_BYTES + NEW_BYTES, FB_BYTES = NW * NT * 64 * 16;
  __shared__ __attribute__((aligned(16))) unsigned char smem[WORK_BYTES > FB_BYTES ? WORK_BYTES : FB_BYTES];
  _Float16* const vt = reinterpret_cast<_Float16*>(smem);
  _Float16* const qs = reinterpret_cast<_Float16*>(smem + VT_BYTES);
  __bf16* const qsb = reinterpret_cast<__bf16*>(smem + VT_BYTES + QS_BYTES);      // the same Q as bf16
  int32_t* const spos = reinterpret_cast<int32_t*>(smem + VT_BYTES + 2 * QS_BYTES);   // -1 = empty slot
  uint8_t* const nrc = smem + VT_BYTES + 2 * QS_BYTES + SPOS_BYTES;                   // S8 new rows' codes
  float* const nrs = reinterpret_cast<float*>(nrc + kMaxSwaNew * D);                  // and their scales
  __shared__ __attribute__((aligned(8))) float ml[NW][16][2];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;

  // grid (8 * 2 * head groups, ceil(nq / 8), splits): blockIdx.x = 8 * (2 * hg
  // + c0) + xcd and q = 8 * blockIdx.y + xcd.  The dispatcher deals linear
  // workgroup ids round-robin to the 8 XCDs and gridDim.x is a multiple of 8,
  // so all workgroups of one query share an XCD (and its L2 for the query's
  // rows, window and Q).  No division: queries past nq exit at once.
  const int xcd = (int)(blockIdx.x & 7), idx = (int)(blockIdx.x >> 3);
  const int q = (int)blockIdx.y * 8 + xcd;
  if (q >= p.nq) return;
  const int c0 = idx & 1, hg = idx >> 1, split = (int)blockIdx.z;
  const int b = p.qn_shift >= 0 ? q >> p.qn_shift : q / p.qn;
  const int j = q - b * p.qn;
  const int h0 = hg * 16;
  const int first_swa = p.swa_len ? p.swa_rows - p.swa_len[b] : 0;
  const int t_end = min(p.n_tiles, (split + 1) * p.tiles_per_split);
  const int sp_end = min(t_end, p.n_sparse_tiles);
  const int tile0 = split * p.tiles_per_split + wave;
  using HV = Halves<D>;
  const int ch[2] = {c0, 1 - c0};                                // column half of each operand half (0 = own)
  // channel of half index o of half ch (SUB is a power of two)
  auto gch = [](int o, int chh) { return HV::BLK * (o / HV::SUB) + HV::SUB * chh + (o % HV::SUB); };

  // Every load below is issued unconditionally (slots, rows and heads that do
  // not exist read zeros through out-of-range buffer offsets), so the compiler
  // can count the loads in flight and waits only for the data it uses.
  constexpr uint32_t kOob = 0xFFFFF000u;            // offset past every buffer
  const int n_fp4 = tile0 < sp_end ? (sp_end - tile0 + NW - 1) / NW : 0;
  const int slot0 = split * p.tiles_per_split * 16;                  // first Top-K slot of this split
  const int n_slots = max(0, sp_end * 16 - slot0);                   // FP4 slots of this split
  const rsrc_t tk_buf = make_rsrc(p.topk + (int64_t)q * p.topk_k, (uint32_t)p.topk_k * 4u);
  // The positions of the wave's first two FP4 tiles go out first (the first
  // gathers depend on them); the whole split's positions follow into LDS, from
  // where each later gather takes its own.  The validity test is applied where
  // a position is used, so nothing waits on these loads here.
  int32_t pos0[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot_i = (tile0 + NW * i) * 16 + n;
    pos0[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(tk_buf, i < n_fp4 && slot_i < p.topk_k ? 4u * (uint32_t)slot_i : kOob, 0, 0);
  }
  // Paged cache (PG): a Top-K position t of sequence b is row
  // block_table[b][t >> page_shift] * page_size + (t & (page_size - 1)) of the
  // whole cache; positions outside [0, T), negative page ids and rows past the
  // cache become -1 (empty).  Positions are translated where they are staged.
  const rsrc_t bt_buf = make_rsrc(PG == 1 ? p.block_table + (int64_t)b * p.max_pages : nullptr,
                                  PG == 1 ? (uint32_t)p.max_pages * 4u : 0u);
  auto to_row = [&](int32_t pos) -> int32_t {
    if constexpr (PG == 0) {
      return pos;
    } else if constexpr (PG == 2) {
      return pos >= 0 && (int64_t)pos < p.cache_rows ? pos : -1;
    } else {
      const bool ok = pos >= 0 && (int64_t)pos < p.T;
      const int32_t page = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
          bt_buf, ok ? 4u * (uint32_t)(pos >> p.page_shift) : kOob, 0, 0);
      const int64_t row = ((int64_t)page << p.page_shift) + (pos & ((1 << p.page_shift) - 1));
      return ok && page >= 0 && row < p.cache_rows ? (int32_t)row : -1;
    }
  };
  auto first_position = [&](int i) {
    const int slot_i = (tile0 + NW * i) * 16 + n;
    return i < n_fp4 && slot_i < p.topk_k ? to_row(pos0[i]) : -1;
  };
  constexpr int SPT = (kMaxTopK + 64 * NW - 1) / (64 * NW);
  int32_t sraw[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sl = (int)threadIdx.x + 64 * NW * i;
    sraw[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(tk_buf, sl < n_slots ? 4u * (uint32_t)(slot0 + sl) : kOob, 0, 0);
  }
  // position of the wave's FP4 tile i (slot n), from LDS
  auto position = [&](int i) { return i < n_fp4 ? spos[(wave + NW * i) * 16 + n] : -1; };

  // ---- Q of the 16 heads (bf16 -> fp16, heads past H read zeros): global
  // loads now, converted into LDS once the first gathers are out; each wave
  // then reads its QK B operand from there
  constexpr int QCH = 16 * D / 8;                   // 8-channel chunks of the Q tile
  constexpr int QPT = (QCH + 64 * NW - 1) / (64 * NW);
  const rsrc_t q_buf = make_rsrc(p.q + ((int64_t)q * p.heads + h0) * D, (uint32_t)(min(16, p.heads - h0) * D * 2));
  u4 qraw[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = threadIdx.x + 64 * NW * i;       // chunk c: head row c / (D / 8), 16 bytes each
    qraw[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(q_buf, c < QCH ? 16u * (uint32_t)c : kOob, 0, 0));
  }
  // S8 with new window rows: wave w takes rows w, w + NW, ... of the
  // sequence's Qn new rows (bf16, 16 bytes per lane; rows past Qn, or no new
  // rows at all, read zeros)
  constexpr int NRW = S8 ? kMaxSwaNew / NW : 1;
  [[maybe_unused]] u4 nraw[NRW];
  if constexpr (S8) {
    const rsrc_t nb_buf = make_rsrc(p.swa_new ? p.swa_new + (int64_t)b * p.qn * D : nullptr,
                                    p.swa_new ? (uint32_t)(p.qn * D * 2) : 0u);
#pragma unroll
    for (int i = 0; i < NRW; ++i) {
      const int r = wave + NW * i;
      nraw[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                           nb_buf, lane < D / 8 ? 16u * (uint32_t)(r * (D / 8) + lane) : kOob, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);                // positions and Q go out before the gathers

  // ---- FP4 rows: the first two gathers go out as soon as their positions
  // are known
  Fp4Src src;
  // the sequence's rows, or (PG) the whole cache
  const int64_t row0 = PG != 0 ? 0 : b * p.T, nrows = PG != 0 ? p.cache_rows : p.T;
  src.codes = make_rsrc(p.codes + row0 * p.codes_stride, (uint32_t)(nrows * p.codes_stride));
  src.scales = make_rsrc(p.scales + row0 * p.scales_stride, (uint32_t)(nrows * p.scales_stride));
  src.cstride = (uint32_t)p.codes_stride;
  src.sstride = (uint32_t)p.scales_stride;
  src.oob = kOob;
  // lane g's block: code bytes BLK/2 * g .. (two halves of SUB/2 bytes each),
  // scale bytes BLK/16 * g .. (D = 512: eight bytes; D = 128: the two bytes
  // 2g, 2g+1, read with the word that holds them)
  src.hcb[0] = HV::SUB / 2 * ch[0]; src.hcb[1] = HV::SUB / 2 * ch[1];
  src.lcb = (uint32_t)(HV::BLK / 2 * g);
  src.lsb = KH == 8 ? 8u * (uint32_t)g : 4u * (uint32_t)(g >> 1);
  // D = 128: the scale of half h is byte 2(g & 1) + ch[h] of the word
  uint32_t psel128[2];
  for (int h = 0; h < 2; ++h) psel128[h] = (uint32_t)(2 * (g & 1) + ch[h]) | (0x0Cu << 8) | (0x0Cu << 16) | (0x0Cu << 24);
  const uint32_t T32 = (uint32_t)nrows;
  Fp4Raw<D> raw[2];
  bool vld[2];
  vld[0] = load_fp4<D>(src, first_position(0), T32, raw[0]);
  vld[1] = load_fp4<D>(src, first_position(1), T32, raw[1]);

#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = threadIdx.x + 64 * NW * i;
    const int hr = c / (D / 8);
    if (c < QCH) {
      *reinterpret_cast<v8h*>(qs + hr * QPITCH + (c % (D / 8)) * 8) = bf16x8_to_half(qraw[i]);
      *reinterpret_cast<u4*>(qsb + hr * QPITCH + (c % (D / 8)) * 8) = qraw[i];
    }
  }
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int sl = (int)threadIdx.x + 64 * NW * i;
    if (sl < n_slots) spos[sl] = slot0 + sl < p.topk_k ? to_row(sraw[i]) : -1;
  }
  if constexpr (PG == 1) {
    // the rows this split's slots name, for the later calls of the group
    // (their Top-K as rows); one workgroup per (query, split) writes them
    if (p.rows_out && hg == 0 && c0 == 0) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int sl = (int)threadIdx.x + 64 * NW * i;
        if (sl < n_slots && slot0 + sl < p.topk_k) p.rows_out[(int64_t)q * p.topk_k + slot0 + sl] = spos[sl];
      }
    }
  }
  if constexpr (S8) {
    if (p.swa_new) {
      // window row swa_rows - Qn + r is the sequence's new row r: encoded as
      // csa2_quantize_swa_fp8 encodes it, for this workgroup's window tiles
      // (from LDS); the first workgroup of the sequence's first query also
      // stores it in its slot of the window cache
      const bool store = j == 0 && hg == 0 && c0 == 0 && split == 0;
#pragma unroll
      for (int i = 0; i < NRW; ++i) {
        const int r = wave + NW * i;
        if (r < p.qn) {
          float sc;
          const u2 c = swa8_encode_row(nraw[i], sc);
          if (lane < D / 8) *reinterpret_cast<u2*>(nrc + r * D + 8 * lane) = c;
          if (lane == 0) nrs[r] = sc;
          if (store) {
            int st = p.swa_start ? p.swa_start[b] : 0;   // ring slot of window row 0
            st = st >= 0 && st < p.swa_rows ? st : 0;
            const int wr = p.swa_rows - p.qn + r;
            const int slot = wr + st >= p.swa_rows ? wr + st - p.swa_rows : wr + st;
            const int64_t crow = (int64_t)b * p.swa_rows + slot;
            if (lane < D / 8) *reinterpret_cast<u2*>(reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(p.swa)) + crow * D + 8 * lane) = c;
            if (lane == 0) const_cast<float*>(p.swa_scale)[crow] = sc;
          }
        }
      }
    }
  }
  __syncthreads();

  v4f o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  _Float16* my = vt + wave * TILE_HALVES;
  const _Float16* vbase = my + (4 * g + (n >> 2)) * PITCH + 4 * (n & 3);   // transposing PV read
  v8h qf[KH];
  auto load_qf = [&](auto map) {
    using M = decltype(map);
#pragma unroll
    for (int k = 0; k < KH; ++k) qf[k] = *reinterpret_cast<const v8h*>(qs + n * QPITCH + gch(M::off(k) + M::LANE * g, ch[0]));
  };

  const int swa_first = tile0 + NW * n_fp4;          // the wave's first window tile
  // ---- window rows (bf16, or 8-bit codes with a scale per row), read
  // through a buffer over this sequence's window (rows outside it read
  // zeros); w holds one 16-row tile
  constexpr uint32_t kSwaBytes = S8 ? 1u : 2u;      // per channel
  u4 w[2][KH];
  bool swa_valid = false;
  uint32_t swa_sc = 0;                               // S8: the lane's row scale (fp32 bits)
  uint32_t swa_so = kOob;                            // S8: byte offset of that scale
  const rsrc_t swa_buf = make_rsrc(reinterpret_cast<const uint8_t*>(p.swa) + (int64_t)b * p.swa_rows * D * kSwaBytes,
                                   (uint32_t)(p.swa_rows * D * kSwaBytes));
  const rsrc_t swa_sbuf = make_rsrc(S8 ? p.swa_scale + (int64_t)b * p.swa_rows : nullptr,
                                    S8 ? (uint32_t)(p.swa_rows * 4) : 0u);
  // byte offset of the lane's first channel within a row (half 0 of block 0;
  // the k-step and the half are added where loaded)
  const uint32_t swa_lane = S8 ? (uint32_t)gch(Fp8Map<D>::LANE * g, 0) : 2u * (uint32_t)gch(InterMap<D>::LANE * g, 0);
  // ring buffer: window row r of the sequence sits in slot (r + start) mod rows
  int swa_st = p.swa_start ? p.swa_start[b] : 0;
  swa_st = swa_st >= 0 && swa_st < p.swa_rows ? swa_st : 0;
  // S8 with new rows: rows swa_rows - Qn .. are not read from the cache (they
  // come from the workgroup's own encoding in LDS)
  const int first_new = S8 && p.swa_new ? p.swa_rows - p.qn : p.swa_rows;
  auto swa_rows = [&](int t) {                      // this lane's row offset of window tile t
    const int wr = (t - p.n_sparse_tiles) * 16 + n;
    const int r = j + wr;
    swa_valid = t < t_end && wr >= 0 && wr < p.window && r >= first_swa && r < p.swa_rows;
    const bool cached = S8 ? swa_valid && r < first_new : swa_valid;
    const int rs = r + swa_st >= p.swa_rows ? r + swa_st - p.swa_rows : r + swa_st;
    swa_so = cached ? 4u * (uint32_t)rs : kOob;
    return (cached ? (uint32_t)rs * (kSwaBytes * D) : kOob) + swa_lane;
  };
  auto load_swa_half = [&](uint32_t ro, int hh) {
    if constexpr (S8) {
#pragma unroll
      for (int i = 0; i < KH / 2; ++i)
        w[hh][i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                              swa_buf, ro + (uint32_t)gch(64 * i, 0),
                                              __builtin_amdgcn_readfirstlane(HV::SUB * ch[hh]), 0));
      if (hh == 0) swa_sc = __builtin_amdgcn_raw_buffer_load_b32(swa_sbuf, swa_so, 0, 0);
    } else {
#pragma unroll
      for (int k = 0; k < KH; ++k)
        w[hh][k] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                              swa_buf, ro + 2u * (uint32_t)gch(InterMap<D>::off(k), 0),
                                              __builtin_amdgcn_readfirstlane(2 * HV::SUB * ch[hh]), 0));
    }
  };
  auto load_swa = [&](int t) {
    const uint32_t ro = swa_rows(t);
    load_swa_half(ro, 0);
    load_swa_half(ro, 1);
  };
  uint32_t swa_ro = kOob;

  // ---- FP4 tiles (runs channel map), two at a time: two tiles' gathers are
  // in flight at all times: tile i + 2 goes into tile i's buffer as soon as
  // tile i's logits are done with it.  Past the wave's last tile the slots are
  // empty: the loads read zeros and such a tile (the second of the last pair)
  // is fully masked, so every pair issues the same loads and the compiler's
  // wait counts stay exact.  The last pair loads the two halves of the wave's
  // first window tile in place of gathers (the same number of loads).
  if (n_fp4 > 0) {
    load_qf(BlockMap<D>{});
    // the other half's Q of k-step k: BlockMap keeps the k-steps of a lane in
    // one block, so they are consecutive
    const _Float16* qol = qs + n * QPITCH + gch(BlockMap<D>::LANE * g, ch[1]);
    _Float16* wrow = my + n * PITCH + BlockMap<D>::LANE * g;
    auto fp4_tile = [&](int u, auto after) {
      Fp4Raw<D>& cur = raw[u];
      // an empty slot read zero codes and scales: finite zeros in V; its
      // logits are masked
      // per half: its scales times 2^-8 (D = 512: four groups of 16 channels
      // per half, k-step k in group k / 2; D = 128: one group per half)
      v2h sc[2][2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if constexpr (KH == 8) {
          const uint32_t sw = ch[hh] ? cur.s[1] : cur.s[0];
          sc[hh][0] = e4m3_pair_s8(sw, 0x0C010C00u);
          sc[hh][1] = e4m3_pair_s8(sw, 0x0C030C02u);
        } else {
          sc[hh][0] = sc[hh][1] = e4m3_pair_s8(cur.s[0], psel128[hh]);
        }
      }
      const bool v = vld[u];
      attend_tile<D, BlockMap<D>, v8h>(
          p,
          [&](int hh, int k) {
            return fp4x8_to_half_s8(cur.w[hh][k], KH == 8 ? sc[hh][k >> 2][(k >> 1) & 1] : sc[hh][0][0]);
          },
          [&](int hh, int k) { return hh == 0 ? qf[k] : *reinterpret_cast<const v8h*>(qol + BlockMap<D>::off(k)); },
          [](v8h kv) { return kv; }, after, v, wrow, vbase, g, o, m_run, l_run);
    };
    int i0 = 0;
    for (; i0 + 2 < n_fp4; i0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) fp4_tile(u, [&]() { vld[u] = load_fp4<D>(src, position(i0 + u + 2), T32, raw[u]); });
    }
    fp4_tile(0, [&]() {
      swa_ro = swa_rows(swa_first);
      load_swa_half(swa_ro, 0);
    });
    fp4_tile(1, [&]() { load_swa_half(swa_ro, 1); });
  }
  if (n_fp4 == 0 && swa_first < t_end) load_swa(swa_first);

  // ---- sliding-window tiles (bf16 rows, interleaved channel map); the
  // first one was loaded during the last FP4 pair (or is loaded here when the
  // wave has no FP4 tile), each next one as soon as the current one's logits
  // are done
  // QK runs on the bf16 rows and the bf16 Q as they are; only the own half
  // becomes fp16 (exactly, inside fp16's range) for PV.  Rows outside the
  // window read as zeros and their logits are masked.
  if constexpr (S8) {
    // 8-bit rows: decoded to fp16 (exact) with the row's scale and contracted
    // like the FP4 rows, against the own half of Q reloaded in this map
    if (swa_first < t_end) {
      load_qf(Fp8Map<D>{});
      _Float16* wrow = my + n * PITCH + Fp8Map<D>::LANE * g;
      for (int t = swa_first; t < t_end; t += NW) {
        // the step's new rows (read as zeros above) from the encoding in LDS
        const int i_new = j + (t - p.n_sparse_tiles) * 16 + n - first_new;
        if (i_new >= 0 && i_new < p.qn && swa_valid) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < KH / 2; ++i)
              w[hh][i] = *reinterpret_cast<const u4*>(nrc + i_new * D + swa_lane + gch(64 * i, 0) + HV::SUB * ch[hh]);
          swa_sc = __float_as_uint(nrs[i_new]);
        }
        const bool v = swa_valid;
        const float sc = __uint_as_float(swa_sc);
        attend_tile<D, Fp8Map<D>, v8h>(
            p, [&](int hh, int k) { return fp8x8_to_half(w[hh][k / 2][2 * (k % 2)], w[hh][k / 2][2 * (k % 2) + 1], sc); },
            [&](int hh, int k) {
              return hh == 0 ? qf[k]
                             : *reinterpret_cast<const v8h*>(qs + n * QPITCH + gch(Fp8Map<D>::off(k) + Fp8Map<D>::LANE * g, ch[1]));
            },
            [](v8h kv) { return kv; }, [&] { if (t + NW < t_end) load_swa(t + NW); }, v, wrow, vbase, g, o, m_run, l_run);
      }
    }
  } else if (swa_first < t_end) {
    v8bf qfb[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k)
      qfb[k] = *reinterpret_cast<const v8bf*>(qsb + n * QPITCH + gch(InterMap<D>::off(k) + InterMap<D>::LANE * g, ch[0]));
    _Float16* wrow = my + n * PITCH + InterMap<D>::LANE * g;
    for (int t = swa_first; t < t_end; t += NW) {
      const bool v = swa_valid;
      attend_tile<D, InterMap<D>, v8bf>(
          p, [&](int hh, int k) { return __builtin_bit_cast(v8bf, w[hh][k]); },
          [&](int hh, int k) {
            return hh == 0 ? qfb[k]
                           : *reinterpret_cast<const v8bf*>(qsb + n * QPITCH + gch(InterMap<D>::off(k) + InterMap<D>::LANE * g, ch[1]));
          },
          [](v8bf kv) { return bf16x8_to_half(__builtin_bit_cast(u4, kv)); }, [&] { if (t + NW < t_end) load_swa(t + NW); }, v, wrow,
          vbase, g, o, m_run, l_run);
    }
  }

  // ---- merge the NW waves: M = max m_w, L = sum f_w l_w, O = sum f_w O_w
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
  if (g == 0) { ml[wave][n][0] = m_run; ml[wave][n][1] = l_tot; }
  __syncthreads();                                  // also: every wave is done with the arena
  // every lane merges head n over the NW waves (independent LDS reads, fixed
  // order); o holds heads 4g + i, whose factors come from lanes 4g + i
  float mw[NW], lw[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float2 v = *reinterpret_cast<const float2*>(&ml[w][n][0]);
    mw[w] = v.x;
    lw[w] = v.y;
  }
  float mx = mw[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, mw[w]);
  float ls = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ls += (mw[w] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - mx) * lw[w];
  const float f_own = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - mx);
  const float inv_own = ls > 0.0f ? 1.0f / ls : 0.0f;
  float fme[4], inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fme[i] = __shfl(f_own, 4 * g + i, 64);
    inv[i] = __shfl(inv_own, 4 * g + i, 64);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[t][i] *= fme[i];

  // every wave leaves its scaled O in a lane-major fp32 buffer over the arena
  // (element (wave, t, lane) holds o[t]); one cooperative pass adds the NW
  // partials in a fixed order
  v4f* fb = reinterpret_cast<v4f*>(smem);
#pragma unroll
  for (int t = 0; t < NT; ++t) fb[(wave * NT + t) * 64 + lane] = o[t];
  __syncthreads();

  // each thread sums the NW partials of tiles t = wave, wave + NW, ... at its
  // own lane, i.e. channel 16t + n of heads 4g .. 4g + 3 (the o layout), so
  // the per-head factors above apply directly
  for (int t = wave; t < NT; t += NW) {
    v4f sum = fb[t * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += fb[(w * NT + t) * 64 + lane];
    const int chg = gch(16 * t + n, c0);
    if (p.splits == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (h0 + 4 * g + i < p.heads) p.out[((int64_t)q * p.heads + h0 + 4 * g + i) * D + chg] = sum[i] * inv[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t pr = ((int64_t)q * p.splits + split) * p.heads + h0 + 4 * g + i;
        if (h0 + 4 * g + i < p.heads) p.opart[pr * D + chg] = sum[i];
      }
    }
  }
  // the split's (max, sum) per head: lane n of wave 0 holds head n's
  if (p.splits > 1 && wave == 0 && g == 0 && c0 == 0 && h0 + n < p.heads) {
    const int64_t pr = ((int64_t)q * p.splits + split) * p.heads + h0 + n;
    p.mlpart[2 * pr] = mx;
    p.mlpart[2 * pr + 1] = ls;
  }
}

// Merge split partials: one workgroup per (query, head), D/4 threads x float4.
template <int D>
__global__ __launch_bounds__(D / 4) void k_attn_combine(AttnParams p) {
  const int64_t qh = blockIdx.x;                    // q * H + h
  const int64_t q = qh / p.heads, h = qh - q * p.heads;
  const int S = p.splits;
  float mx = -__builtin_inff();
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.mlpart[2 * ((q * S + s) * p.heads + h)]);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const int64_t pr = (q * S + s) * p.heads + h;
    const float ms = p.mlpart[2 * pr];
    const float f = (ms == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms - mx);
    L += f * p.mlpart[2 * pr + 1];
    const float4 v = reinterpret_cast<const float4*>(p.opart + pr * D)[threadIdx.x];
    acc.x += f * v.x; acc.y += f * v.y; acc.z += f * v.z; acc.w += f * v.w;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  reinterpret_cast<float4*>(p.out + qh * D)[threadIdx.x] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

hipError_t launch_attn(const AttnParams& p, int nq, int dim, int waves, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  const int ngroups = (p.heads + 15) / 16;
  const dim3 grid((unsigned)(16 * ngroups), (unsigned)((nq + 7) / 8), (unsigned)p.splits);
#define CSA2_ATTN_CASE(D, NW)                                                                 \
  if (dim == D && waves == NW) {                                                              \
    if (p.block_table) {                                                                      \
      if (p.swa_fp8) hipLaunchKernelGGL((k_attn<D, NW, true, 1>), grid, dim3(64 * NW), 0, st, p); \
      else hipLaunchKernelGGL((k_attn<D, NW, false, 1>), grid, dim3(64 * NW), 0, st, p);        \
    } else if (p.rows_in) {                                                                   \
      if (p.swa_fp8) hipLaunchKernelGGL((k_attn<D, NW, true, 2>), grid, dim3(64 * NW), 0, st, p); \
      else hipLaunchKernelGGL((k_attn<D, NW, false, 2>), grid, dim3(64 * NW), 0, st, p);        \
    } else {                                                                                  \
      if (p.swa_fp8) hipLaunchKernelGGL((k_attn<D, NW, true, 0>), grid, dim3(64 * NW), 0, st, p); \
      else hipLaunchKernelGGL((k_attn<D, NW, false, 0>), grid, dim3(64 * NW), 0, st, p);        \
    }                                                                                         \
    if (p.splits > 1) hipLaunchKernelGGL(k_attn_combine<D>, dim3(nq * p.heads), dim3(D / 4), 0, st, p); \
    return hipGetLastError();                                                                 \
  }
  CSA2_ATTN_CASE(512, 4) CSA2_ATTN_CASE(512, 8) CSA2_ATTN_CASE(128, 4) CSA2_ATTN_CASE(128, 8)
#undef CSA2_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace csa2
