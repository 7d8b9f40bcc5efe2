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
//  * workgroup = (query, group of 16 heads, split of the tile list); its 4
//    waves take every 4th 16-entry tile of the split and merge their
//    (max, sum, O) states through LDS at the end.  When the tile list is split
//    over several workgroups, a second kernel merges the partial states.
//  * per tile a wave gathers 16 entries: lane (e = lane % 16, quarter =
//    lane / 16) loads entry e's channels [D/4*quarter, D/4*(quarter+1)):
//    D/8 FP4 code bytes + D/64 E4M3 scales, or D/4 bf16 SWA values, and
//    turns them into fp16 in registers (FP4 values are exact in fp16).
//  * QK^T: MFMA 16x16x32 f16 with the entries as A rows and the 16 heads as
//    B columns; each lane's own dequantised channels are its A fragment (the
//    contraction only needs A and B to agree on the channel order, and Q is
//    loaded in the same order).  The result holds entries 4*(lane/16)+i of
//    head lane%16 -- exactly the A-operand layout of the PV MFMA, so the
//    probabilities never leave registers.
//  * PV: MFMA 16x16x16 f16 over the 16 entries; the V operand needs 4 entries
//    of one channel per lane, which one transposing LDS read per 16 channels
//    delivers from the wave's fp16 tile.
//  * the next tile's gather is issued before the current tile is processed.
// Q and SWA rows go bf16 -> fp16 unscaled, which is exact for magnitudes in
// [2^-14, 65504] (bf16 carries 8 significant bits, fp16 11), so QK^T is exact
// up to fp32 accumulation; sm_scale * log2(e) multiplies the fp32 logits and
// the softmax uses exp2.
#include "common.h"

namespace csa2 {

CSA2_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4s __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// output lane i, slot r receives element (i % 4) of the 4 consecutive halves
// that lane 4r + i/4 of the group addresses.
CSA2_DEV v4h lds_read_tr16(const _Float16* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(v4h, r);
}

// max over lanes {l, l^16, l^32, l^48}: gfx950 permlane swaps (no LDS traffic);
// permlane16_swap(x, x) yields the values of lanes l and l^16, the 32 variant
// those of l and l^32
CSA2_DEV float max_over_quarters(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int SEL>
CSA2_DEV _Float16 scale_half(uint32_t w) { return e4m3_to_half<SEL>(w); }

CSA2_DEV _Float16 scale_sel(uint32_t w, int sel) {
  switch (sel & 3) {            // sel is a constant after unrolling
    case 0: return scale_half<0>(w);
    case 1: return scale_half<1>(w);
    case 2: return scale_half<2>(w);
    default: return scale_half<3>(w);
  }
}

// FP4 tile data of this lane (entry lane%16, channel quarter lane/16):
// D/8 code bytes and D/64 scale bytes.
template <int D>
struct Fp4Raw {
  u4 c[D / 128];
  uint32_t s[2];
};

template <int D>
CSA2_DEV bool load_fp4(const AttnParams& p, int32_t pos, int64_t b, int g, Fp4Raw<D>& r) {
  constexpr int CB = D / 8, SB = D / 64;
  const bool valid = pos >= 0 && (int64_t)pos < p.T;
  const int64_t row = b * p.T + (valid ? pos : 0);
  const uint8_t* cp = p.codes + row * p.codes_stride + CB * g;
  const uint8_t* sp = p.scales + row * p.scales_stride + SB * g;
#pragma unroll
  for (int c = 0; c < D / 128; ++c) r.c[c] = *reinterpret_cast<const u4*>(cp + 16 * c);
  if constexpr (SB == 8) {
    const u2 w = *reinterpret_cast<const u2*>(sp);
    r.s[0] = w[0];
    r.s[1] = w[1];
  } else {
    r.s[0] = *reinterpret_cast<const uint16_t*>(sp);
    r.s[1] = 0u;
  }
  return valid;
}

// LDS tiles are padded rows of D + 8 halves: consecutive rows start 4 banks
// apart, so the 16-byte staging writes and Q reads (16 rows, same column) and
// the transposing V reads stay within a few bank groups, and every address is
// a per-lane base plus a compile-time offset.
template <int D, typename KV>
CSA2_DEV void attend_tile(const AttnParams& p, KV kvf, bool valid, const _Float16* qbase, _Float16* wbase,
                          const _Float16* vbase, int g, v4f (&o)[D / 16], float& m_run, float& l_run) {
  constexpr int KS = D / 32, NT = D / 16;
  constexpr int NA = KS >= 4 ? 4 : KS;      // independent MFMA accumulation chains
  v4f accs[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) accs[a] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const v8h kv = kvf(ks);
    const v8h qv = *reinterpret_cast<const v8h*>(qbase + 8 * ks);
    accs[ks % NA] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qv, accs[ks % NA], 0, 0, 0);
    *reinterpret_cast<v8h*>(wbase + 8 * ks) = kv;
  }
  v4f acc = accs[0];
#pragma unroll
  for (int a = 1; a < NA; ++a) acc += accs[a];

  // online softmax (head = lane % 16, entries 4g..4g+3).  The reference max
  // only moves when a tile's max exceeds it by more than 2^8, so O is rarely
  // rescaled; probabilities stay <= 256, fine for fp16.
  const uint64_t vm = __ballot(valid);
  float s4[4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s4[i] = ((vm >> (4 * g + i)) & 1ull) ? acc[i] * p.qscale : -__builtin_inff();
    tmax = fmaxf(tmax, s4[i]);
  }
  tmax = max_over_quarters(tmax);
  const bool grow = tmax > m_run + 8.0f;
  float alpha = 1.0f;
  if (grow) {
    alpha = __builtin_amdgcn_exp2f(m_run - tmax);
    m_run = tmax;
  }
  v4h pa;
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 ph = (s4[i] == -__builtin_inff()) ? (_Float16)0.0f : (_Float16)__builtin_amdgcn_exp2f(s4[i] - m_run);
    pa[i] = ph;
    psum += (float)ph;          // normalise with the probabilities actually used
  }
  l_run = l_run * alpha + psum;
  if (__any(grow)) {
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

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn(AttnParams p) {
  constexpr int KS = D / 32;        // QK k-steps; each lane holds 8*KS = D/4 channels
  constexpr int NT = D / 16;        // PV output tiles of 16 channels
  constexpr int PITCH = D + 8;      // LDS row pitch in halves
  __shared__ __attribute__((aligned(16))) _Float16 vt[NW * 16 * PITCH];  // per-wave V tiles
  __shared__ __attribute__((aligned(16))) _Float16 qs[16 * PITCH];       // Q of the 16 heads

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ngroups = (p.heads + 15) >> 4;
  const int hg = blockIdx.x % ngroups, split = blockIdx.x / ngroups;
  const int64_t q = blockIdx.y;
  const int64_t b = q / p.qn;
  const int j = (int)(q - b * p.qn);
  const int h0 = hg * 16;
  const int first_swa = p.swa_len ? p.swa_rows - p.swa_len[b] : 0;
  const int t_end = min(p.n_tiles, (split + 1) * p.tiles_per_split);
  const int sp_end = min(t_end, p.n_sparse_tiles);
  int tile = split * p.tiles_per_split + wave;

  // Top-K positions of this wave's first batch of FP4 tiles go out before the
  // Q staging so the latencies overlap (a tile's gather then needs no
  // dependent index load)
  constexpr int PB = 8;                             // FP4 tiles per position batch
  const int n_fp4 = tile < sp_end ? (sp_end - tile + NW - 1) / NW : 0;
  auto load_positions = [&](int first, int32_t (&pos)[PB]) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int ti = tile + NW * (first + i);
      const int slot = ti * 16 + n;
      pos[i] = (first + i < n_fp4 && slot < p.topk_k) ? p.topk[q * p.topk_k + slot] : -1;
    }
  };
  int32_t pos[PB];
  load_positions(0, pos);

  // ---- stage Q (16 heads x D, bf16 -> fp16 unscaled, exact in fp16's normal
  // range) in LDS; every wave reads its B operand from there.  The Q loads and
  // the first FP4 gather are both in flight before either is waited on.
  constexpr int QCH = 16 * D / 8;                 // 8-half chunks of the Q tile
  constexpr int QPT = (QCH + 64 * NW - 1) / (64 * NW);
  u4 qraw[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = threadIdx.x + 64 * NW * i;
    const int hr = c / (D / 8), h = h0 + hr;
    if (c < QCH) qraw[i] = *reinterpret_cast<const u4*>(p.q + (q * p.heads + (h < p.heads ? h : 0)) * D +
                                                         (c % (D / 8)) * 8);
  }
  Fp4Raw<D> raw;
  bool valid = n_fp4 > 0 ? load_fp4<D>(p, pos[0], b, g, raw) : false;
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int c = threadIdx.x + 64 * NW * i;
    const int hr = c / (D / 8);
    v8h f = bf16x8_to_half(qraw[i]);
    if (h0 + hr >= p.heads) f = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    if (c < QCH) *reinterpret_cast<v8h*>(qs + hr * PITCH + (c % (D / 8)) * 8) = f;
  }
  __syncthreads();

  v4f o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  _Float16* my = vt + wave * 16 * PITCH;
  _Float16* wbase = my + n * PITCH + (D / 4) * g;                  // staging: entry n, quarter g
  const _Float16* vbase = my + (4 * g + (n >> 2)) * PITCH + 4 * (n & 3);   // transposing PV read
  const _Float16* qbase = qs + n * PITCH + (D / 4) * g;            // QK B operand: head n
  const v8h zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  // ---- FP4 tiles: positions in batches of PB, next gather in flight while
  // the current tile is processed
  for (int first = 0; first < n_fp4; first += PB) {
    if (first > 0) {
      load_positions(first, pos);
      valid = load_fp4<D>(p, pos[0], b, g, raw);
    }
    const int cnt = min(PB, n_fp4 - first);
#pragma unroll 1
    for (int i = 0; i < cnt; ++i) {
#pragma unroll
      for (int k = 0; k + 1 < PB; ++k) pos[k] = pos[k + 1];   // pos[0] = next tile
      const Fp4Raw<D> cur = raw;
      const bool cur_valid = valid;
      if (i + 1 < cnt) valid = load_fp4<D>(p, pos[0], b, g, raw);
      // an empty slot gets scale 0: finite zeros in V, and its logits are masked
      _Float16 sc[KS / 2];
#pragma unroll
      for (int gi = 0; gi < KS / 2; ++gi) sc[gi] = cur_valid ? scale_sel(cur.s[gi >> 2], gi & 3) : (_Float16)0.0f;
      attend_tile<D>(p, [&](int ks) { return fp4x8_to_half(cur.c[ks >> 2][ks & 3], sc[ks >> 1]); },
                     cur_valid, qbase, wbase, vbase, g, o, m_run, l_run);
    }
  }
  tile += NW * n_fp4;
  // ---- sliding-window tiles (bf16 rows)
  for (; tile < t_end; tile += NW) {
    const int wr = (tile - p.n_sparse_tiles) * 16 + n;
    const int r = j + wr;
    const bool v = wr < p.window && r >= first_swa && r < p.swa_rows;
    const uint16_t* rp = p.swa + ((b * p.swa_rows + (v ? r : 0)) * D + (D / 4) * g);
    u4 w[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = *reinterpret_cast<const u4*>(rp + 8 * ks);
    attend_tile<D>(p, [&](int ks) { return v ? bf16x8_to_half(w[ks]) : zero8; }, v, qbase, wbase, vbase, g,
                   o, m_run, l_run);
  }

  // ---- merge the NW waves: M = max m_w, L = sum f_w l_w, O = sum f_w O_w
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
  __syncthreads();                                  // every wave is done with the Q tile
  float (*ml)[16][2] = reinterpret_cast<float (*)[16][2]>(qs);
  if (g == 0) { ml[wave][n][0] = m_run; ml[wave][n][1] = l_tot; }
  __syncthreads();
  float M[4], L[4], fme[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    float mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, ml[w][hh][0]);
    float ls = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = ml[w][hh][0];
      ls += (mw == -__builtin_inff()) ? 0.0f : exp2f(mw - mx) * ml[w][hh][1];
    }
    const float mme = ml[wave][hh][0];
    M[i] = mx;
    L[i] = ls;
    fme[i] = (mme == -__builtin_inff()) ? 0.0f : exp2f(mme - mx);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[t][i] *= fme[i];

  // pairwise tree in a fixed order through a lane-major fp32 buffer
  // (element (slot, t, lane) holds o[t] of one wave); reuses the tile buffers
  v4f* fb = reinterpret_cast<v4f*>(vt);
#pragma unroll
  for (int r = 1; r < NW; r <<= 1) {
    if ((wave & (2 * r - 1)) == r) {
      const int slot = wave / (2 * r);
#pragma unroll
      for (int t = 0; t < NT; ++t) fb[(slot * NT + t) * 64 + lane] = o[t];
    }
    __syncthreads();
    if ((wave & (2 * r - 1)) == 0) {
      const int slot = wave / (2 * r);
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t] += fb[(slot * NT + t) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      if (hh >= p.heads) continue;
      const float inv = L[i] > 0.0f ? 1.0f / L[i] : 0.0f;
      float* dst = p.out + (q * p.heads + hh) * D + n;
#pragma unroll
      for (int t = 0; t < NT; ++t) dst[16 * t] = o[t][i] * inv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      if (hh >= p.heads) continue;
      const int64_t pr = (q * p.splits + split) * p.heads + hh;
      float* dst = p.opart + pr * D + n;
#pragma unroll
      for (int t = 0; t < NT; ++t) dst[16 * t] = o[t][i];
      if (n == 0) { p.mlpart[2 * pr] = M[i]; p.mlpart[2 * pr + 1] = L[i]; }
    }
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
    const float f = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - mx);
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
  const dim3 grid(ngroups * p.splits, nq);
#define CSA2_ATTN_CASE(D, NW)                                                                 \
  if (dim == D && waves == NW) {                                                              \
    hipLaunchKernelGGL((k_attn<D, NW>), grid, dim3(64 * NW), 0, st, p);                       \
    if (p.splits > 1) hipLaunchKernelGGL(k_attn_combine<D>, dim3(nq * p.heads), dim3(D / 4), 0, st, p); \
    return hipGetLastError();                                                                 \
  }
  CSA2_ATTN_CASE(512, 4) CSA2_ATTN_CASE(512, 8) CSA2_ATTN_CASE(128, 4) CSA2_ATTN_CASE(128, 8)
#undef CSA2_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace csa2
