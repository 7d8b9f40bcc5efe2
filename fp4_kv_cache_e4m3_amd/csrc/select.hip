// Selection stages of the CSA2 hierarchical indexer for gfx950: top-2,048
// blocks (the pool) and Top-512 positions of a Full layer, and the Reindex
// rescoring of the pool with its selection.
//
// Method: DeepSeek-V4.1-Flash pages, ai-maestro.online section "Compressed
// Sparse Attention 2": a Full layer selects fresh Top-512 indices through a
// candidate pool of up to 16,384 positions (2,048 blocks of eight tokens);
// Reindex layers rescore that pool with their own indexer Q instead of the
// whole context.  Ranking by (score desc, index asc); outputs ascending.
//
// Design (gfx950, wave64):
//  * Select: one 1024-thread workgroup per query.  A radix select over the
//    offset key - kmin (12-, 12- and up to 8-bit digits; histograms cleared
//    once up front; one wave finds each digit with two DPP scans) gives the
//    K-th largest key and how many keys equal to it are taken; a packed
//    block scan (count above, count equal) emits the winners in ascending
//    index order, ties to the lowest index.  Atomics only count, never decide
//    membership, so the output is deterministic.
//  * Full: the Top-512 positions lie in the top 512 blocks, so the first
//    block pass also yields a key floor that prunes the candidate blocks; their
//    token keys are gathered while the pool select finishes.
//  * Reindex: the scan's MFMA scoring on gathered pool blocks (2 blocks = one
//    16-token tile), then the same selection.
#include "quant_dev.h"

namespace csa2 {

// ============================================================== select
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kDigitBins = 4096;                 // 12-bit digits: bits 31..20, 19..8, then 7..0
constexpr int kSelHists = 6;                     // 3 passes x 2 selections, cleared once

struct SelShared {
  alignas(16) uint32_t hist[kSelHists][kDigitBins];
  uint32_t bc[4];
  alignas(16) uint32_t wsum[kSelWaves];
  uint32_t wmin[kSelWaves];
  uint32_t wcnt[kSelWaves];
  int32_t pool[kPoolBlocks];
  int32_t sbpool[kPoolBlocks];                   // chosen super-blocks (large pools only)
  int32_t cand[kSelThreads];                     // Top-512 candidate blocks (Full select, fast path)
  uint32_t pkey[kPoolBlocks];                    // keys of the pool's blocks (pool-only select)
};

// inclusive prefix sum over the 64 lanes with DPP (row shifts inside 16-lane
// rows, then row broadcasts across rows); no LDS traffic
CSA2_DEV uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// exclusive prefix sum over the workgroup (thread order), plus the total:
// wave scans, then every thread adds the totals of the lower waves (broadcast
// LDS reads); the second barrier keeps wsum intact until all have read it
CSA2_DEV uint32_t block_excl_scan_total(uint32_t v, SelShared& sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0u, all = 0u;
  const u4* w4 = reinterpret_cast<const u4*>(sh.wsum);
#pragma unroll
  for (int i = 0; i < kSelWaves / 4; ++i) {
    const u4 x = w4[i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      before += 4 * i + c < wave ? x[c] : 0u;
      all += x[c];
    }
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

CSA2_DEV uint32_t block_excl_scan(uint32_t v, SelShared& sh) {
  uint32_t total;
  return block_excl_scan_total(v, sh, total);
}

// +1 on counter `bin`.  When every active lane of the wave hits the same bin
// (ties, concentrated scores) one lane adds the whole count, so a repeated
// digit does not serialise 64 LDS atomics on one address.  The leader's bin
// comes from readfirstlane (a scalar register), not a cross-lane LDS shuffle.
CSA2_DEV void hist_inc(uint32_t* hist, uint32_t bin, bool active) {
  if (active) {
    const uint32_t lb = __builtin_amdgcn_readfirstlane(bin);
    const uint64_t act = __ballot(1);
    const uint64_t same = __ballot(bin == lb);
    if (same == act) {
      const uint32_t lane = __builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
      if (lane == 0) atomicAdd(&hist[lb], (uint32_t)__popcll(act));
    } else {
      atomicAdd(&hist[bin], 1u);
    }
  }
}

// Digit d of an NB-bin histogram (NB = 4096 or 256) with
// above(d) < k <= above(d) + count(d), where above(d) counts larger digits;
// 1 <= k <= the histogram's total.  One wave searches: lane l sums the NB/64
// bins [NB - (NB/64)(l+1), NB - (NB/64) l), so lane order is descending digit
// order; a DPP scan over the lane sums finds the lane whose bins hold the k-th
// key, and a second scan over that lane's bins (one per lane, highest first)
// finds the bin.
template <int NB>
CSA2_DEV void wave_hist_find(const uint32_t* hist, uint32_t k, uint32_t& digit, uint32_t& above) {
  constexpr int BPL = NB / 64;
  static_assert(BPL == 64 || BPL == 4, "4096- or 256-bin histograms");
  const int lane = threadIdx.x & 63;
  const u4* h4 = reinterpret_cast<const u4*>(hist + NB - BPL * (lane + 1));
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPL / 4; ++i) {
    const u4 v = h4[i];
    sum += (v[0] + v[1]) + (v[2] + v[3]);
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t ex = incl - sum;
  const int L = (int)__builtin_ctzll(__ballot(ex < k && k <= incl));
  const uint32_t exL = (uint32_t)__builtin_amdgcn_readlane((int)ex, L);
  const int bin = NB - BPL * L - 1 - min(lane, BPL - 1);
  const uint32_t c = lane < BPL ? hist[bin] : 0u;
  const uint32_t incl2 = exL + wave_incl_scan(c);
  const int M = (int)__builtin_ctzll(__ballot(lane < BPL && incl2 - c < k && k <= incl2));
  digit = (uint32_t)__builtin_amdgcn_readlane(bin, M);
  above = (uint32_t)__builtin_amdgcn_readlane((int)(incl2 - c), M);
}

// wave_hist_find in wave 0, the result broadcast through LDS (the other waves
// only wait at the barrier).  sh.bc is next written after the workgroup has
// passed at least one more barrier, so one barrier suffices here.
template <int NB>
CSA2_DEV void hist_find(const uint32_t* hist, uint32_t k, SelShared& sh, uint32_t& digit, uint32_t& above) {
  if (threadIdx.x < 64) {
    uint32_t d, a;
    wave_hist_find<NB>(hist, k, d, a);
    if (threadIdx.x == 0) { sh.bc[0] = d; sh.bc[1] = a; }
  }
  __syncthreads();
  digit = sh.bc[0];
  above = sh.bc[1];
}

// inclusive max-scan over the 64 lanes with DPP (lanes outside a row read 0,
// which is neutral for unsigned max)
CSA2_DEV uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true));   // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true));   // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true));   // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true));   // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return x;
}

// Largest and smallest nonzero key and the number of nonzero keys over the
// workgroup (kmin = ~0, kmax = 0 when there is none); the smallest is taken as
// the largest complement.
template <int KPT, typename Get>
CSA2_DEV void key_stats(Get get, SelShared& sh, uint32_t& kmin, uint32_t& kmax, uint32_t& count) {
  uint32_t mx = 0u, mnc = 0u, cnt = 0u;
#pragma unroll 16
  for (int j = 0; j < KPT; ++j) {
    const uint32_t k = get(j);
    mx = max(mx, k);
    mnc = max(mnc, k != 0u ? ~k : 0u);
    cnt += k != 0u ? 1u : 0u;
  }
  mx = __builtin_amdgcn_readlane(wave_incl_max(mx), 63);
  mnc = __builtin_amdgcn_readlane(wave_incl_max(mnc), 63);
  cnt = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sh.wsum[wave] = mx; sh.wmin[wave] = mnc; sh.wcnt[wave] = cnt; }
  __syncthreads();
  mx = 0u; mnc = 0u; cnt = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) { mx = max(mx, sh.wsum[w]); mnc = max(mnc, sh.wmin[w]); cnt += sh.wcnt[w]; }
  __syncthreads();
  kmax = mx;
  kmin = ~mnc;
  count = cnt;
}

// K-th largest key among nonzero keys (1 <= K <= #nonzero): tau, the key
// value, and how many keys equal to tau belong to the top K.  kmin / kmax are
// the smallest / largest nonzero key.  Radix passes run on the offset
// r = key - kmin, whose width w is known from the key range: the first pass
// takes its top 12 bits (so the keys spread over all 4096 bins whatever their
// magnitude, and equal digits rarely collide in the LDS atomics), a second
// pass the next up to 12 bits, a third the remaining up to 8.  Histograms
// h[0..2] are pre-cleared.  get(j) returns this thread's j-th key (j < KPT);
// small KPT keeps keys in registers, large KPT re-reads them each pass.
// radix_first runs the first pass and, when kx > 0, also returns thr_x, the
// smallest key whose first digit is that of the kx-th largest key: every key
// ranked within the top kx is >= thr_x.  radix_rest finishes the select.
struct RadixState {
  uint32_t kmin;
  int s1, b2, s2;           // bits below the first digit, second digit width, bits below it
  uint32_t d1, kk;          // first digit, rank left inside it
};

template <int KPT, typename Get>
CSA2_DEV RadixState radix_first(Get get, uint32_t K, uint32_t kmin, uint32_t kmax, SelShared& sh,
                                uint32_t (*h)[kDigitBins], uint32_t kx, uint32_t& thr_x) {
  RadixState st;
  const uint32_t range = kmax - kmin;
  const int width = range == 0u ? 0 : 32 - __builtin_clz(range);
  st.kmin = kmin;
  st.s1 = width > 12 ? width - 12 : 0;
  st.b2 = st.s1 > 12 ? 12 : st.s1;
  st.s2 = st.s1 - st.b2;
#pragma unroll 16
  for (int j = 0; j < KPT; ++j) {
    const uint32_t k = get(j);
    hist_inc(h[0], (k - kmin) >> st.s1, k != 0u);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t d, a, dx = 0u, ax;
    wave_hist_find<kDigitBins>(h[0], K, d, a);
    if (kx > 0u) wave_hist_find<kDigitBins>(h[0], kx, dx, ax);
    if (threadIdx.x == 0) { sh.bc[0] = d; sh.bc[1] = a; sh.bc[2] = dx; }
  }
  __syncthreads();
  st.d1 = sh.bc[0];
  st.kk = K - sh.bc[1];
  thr_x = kmin + (sh.bc[2] << st.s1);
  return st;
}

template <int KPT, typename Get>
CSA2_DEV void radix_rest(Get get, const RadixState& st, SelShared& sh, uint32_t (*h)[kDigitBins], uint32_t& tau,
                         uint32_t& need) {
  const uint32_t kmin = st.kmin;
  const int s1 = st.s1, b2 = st.b2, s2 = st.s2;
  uint32_t kk = st.kk;
  uint32_t pre = st.d1;                                        // known high bits of the offset
  if (b2 > 0) {
    const uint32_t m2 = (1u << b2) - 1u;
#pragma unroll 16
    for (int j = 0; j < KPT; ++j) {
      const uint32_t k = get(j);
      const uint32_t r = k - kmin;
      hist_inc(h[1], (r >> s2) & m2, k != 0u && (r >> s1) == st.d1);
    }
    __syncthreads();
    uint32_t d2, a2;
    hist_find<kDigitBins>(h[1], kk, sh, d2, a2);
    kk -= a2;
    pre = (pre << b2) | d2;
  }
  if (s2 > 0) {
    const uint32_t m3 = (1u << s2) - 1u;
#pragma unroll 16
    for (int j = 0; j < KPT; ++j) {
      const uint32_t k = get(j);
      const uint32_t r = k - kmin;
      hist_inc(h[2], r & m3, k != 0u && (r >> s2) == pre);
    }
    __syncthreads();
    uint32_t d3, a3;
    hist_find<256>(h[2], kk, sh, d3, a3);
    kk -= a3;
    pre = (pre << s2) | d3;
  }
  tau = kmin + pre;
  need = kk;
}

template <int KPT, typename Get>
CSA2_DEV void radix_select(Get get, uint32_t K, uint32_t kmin, uint32_t kmax, SelShared& sh,
                           uint32_t (*h)[kDigitBins], uint32_t& tau, uint32_t& need) {
  uint32_t unused;
  const RadixState st = radix_first<KPT>(get, K, kmin, kmax, sh, h, 0u, unused);
  radix_rest<KPT>(get, st, sh, h, tau, need);
}

CSA2_DEV void hists_clear(SelShared& sh) {
  u4* hp = reinterpret_cast<u4*>(&sh.hist[0][0]);
  constexpr int n4 = kSelHists * kDigitBins / 4;
  for (int i = threadIdx.x; i < n4; i += kSelThreads) hp[i] = u4{0u, 0u, 0u, 0u};
}

// Emit the indices of the top-K keys in ascending index order.  Thread t owns
// indices [t*KPT, t*KPT + KPT); emit(o, j) writes output slot o for local j.
template <int KPT, typename Get, typename Emit>
CSA2_DEV void compact_topk(Get get, uint32_t tau, uint32_t need, SelShared& sh, Emit emit) {
  uint32_t ngt = 0, neq = 0;
#pragma unroll 16
  for (int j = 0; j < KPT; ++j) {
    const uint32_t k = get(j);
    ngt += k > tau ? 1u : 0u;
    neq += k == tau ? 1u : 0u;
  }
  const uint32_t ex = block_excl_scan((ngt << 16) | neq, sh);
  const uint32_t gt_before = ex >> 16, eq_before = ex & 0xFFFFu;
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t r = eq_before;
#pragma unroll 16
  for (int j = 0; j < KPT; ++j) {
    const uint32_t k = get(j);
    if (k > tau) {
      emit(pos++, j);
    } else if (k == tau) {
      if (r < need) emit(pos++, j);
      ++r;
    }
  }
}

// Candidate step shared by Full and Reindex: candidate c = 8*slot + r refers
// to position 8*pool[slot] + r; keys[c] is its score key (0 = not a candidate).
// known_k2 > 0: the caller knows K2 = min(512, #nonzero keys), a lower bound
// kmin of the nonzero keys and an upper bound kmax of all keys, and the
// statistics pass is skipped (the radix digits then span [kmin, kmax]).
template <int KPT2>
CSA2_DEV void select_positions(const uint32_t (&key)[KPT2], SelShared& sh, const int32_t* pool_slots,
                               int32_t* topk_out, uint32_t known_k2 = 0u, uint32_t known_kmin = 0u,
                               uint32_t known_kmax = 0u) {
  auto get = [&](int j) { return key[j]; };
  uint32_t kmin = known_kmin, kmax = known_kmax, nvalid = known_k2;
  if (known_k2 == 0u) key_stats<KPT2>(get, sh, kmin, kmax, nvalid);
  const uint32_t K2 = min(nvalid, (uint32_t)kTopK);
  if (K2 > 0) {
    uint32_t tau, need;
    radix_select<KPT2>(get, K2, kmin, kmax, sh, &sh.hist[3], tau, need);
    const int base = threadIdx.x * KPT2;
    compact_topk<KPT2>(get, tau, need, sh, [&](uint32_t o, int j) {
      const int c = base + j;
      topk_out[o] = pool_slots[c >> 3] * kBlock + (c & 7);
    });
  }
  for (int i = K2 + threadIdx.x; i < kTopK; i += kSelThreads) topk_out[i] = -1;
}

// Full layer: pool of top-2048 blocks, then Top-512 of the pool's positions.
template <int KPT1>
__global__ __launch_bounds__(kSelThreads) void k_select_full(SelectParams p) {
  constexpr int KPT2 = kPoolPositions / kSelThreads;   // 16
  __shared__ SelShared sh;
  // workgroups past the selection quantise the step's new main-KV rows
  if ((int)blockIdx.x >= p.sel_wgs) {
    quantize_job_thread(p.qj, (int64_t)(blockIdx.x - p.sel_wgs) * kSelThreads + threadIdx.x);
    return;
  }
  // p.roles == 2: two workgroups per query, role 0 selects and writes the
  // pool, role 1 the Top-512 (from the pruned candidates, or -- when those are
  // too many -- through its own copy of the pool); p.roles == 1: one
  // workgroup does both (role 2)
  const int64_t q = p.roles == 2 ? (int64_t)(blockIdx.x >> 1) : (int64_t)blockIdx.x;
  const int role = p.roles == 2 ? (int)(blockIdx.x & 1) : 2;
  // the histograms are cleared while the first keys are in flight
  int64_t nv = p.nvis ? (int64_t)p.nvis[q] : p.T;
  nv = max((int64_t)0, min(nv, p.T));
  const int64_t nb = (nv + kBlock - 1) / kBlock;
  const uint32_t K1 = (uint32_t)min(nb, (int64_t)kPoolBlocks);

  // ---- step 1: top blocks (keys in registers when they fit, else re-read)
  const int64_t base1 = (int64_t)threadIdx.x * KPT1;
  const uint32_t* bk = p.bkeys + q * p.bk_stride;
  int ncand = -1;                       // >= 0: Top-512 candidates are sh.cand[0..ncand), keys in ckey
  uint32_t ckey[kBlock] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  // for the candidates' select: how many positions it takes, a floor of the
  // candidate keys and the largest key (the best block's maximum)
  uint32_t c_k2 = 0u, c_kmin = 0u, c_kmax = 0u;
  if constexpr (KPT1 <= 16) {
    uint32_t bkey[KPT1];
    if (base1 + KPT1 <= nb) {                 // whole run visible: 16-byte loads
#pragma unroll
      for (int j = 0; j < KPT1; j += 4) {
        const u4 v = *reinterpret_cast<const u4*>(bk + base1 + j);
        bkey[j] = v[0]; bkey[j + 1] = v[1]; bkey[j + 2] = v[2]; bkey[j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT1; ++j) bkey[j] = base1 + j < nb ? bk[base1 + j] : 0u;
    }
    hists_clear(sh);
    __syncthreads();
    auto get = [&](int j) { return bkey[j]; };
    if (K1 > 0) {
      uint32_t tau, need, kmin, kmax, cnt, thr;
      key_stats<KPT1>(get, sh, kmin, kmax, cnt);
      const RadixState st = radix_first<KPT1>(get, K1, kmin, kmax, sh, &sh.hist[0], min(K1, (uint32_t)kTopK), thr);
      // Top-512 candidates: every block ranked above the block of a selected
      // position holds a position ranked above it, so the Top-512 positions
      // lie in the top 512 blocks, and those have keys >= thr.  When at most
      // one block per thread passes, their ids (ascending) go to sh.cand and
      // their token keys are gathered now, while the pool select finishes.
      uint32_t mine = 0, ntot = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < KPT1; ++j) mine += bkey[j] >= thr ? 1u : 0u;     // thr >= kmin >= 1: key 0 fails
      uint32_t o = role != 0 ? block_excl_scan_total(mine, sh, ntot) : 0u;
      if (ntot <= (uint32_t)kSelThreads) {
#pragma unroll
        for (int j = 0; j < KPT1; ++j)
          if (bkey[j] >= thr) sh.cand[o++] = (int32_t)(base1 + j);
        __syncthreads();
        ncand = (int)ntot;
        if ((int)threadIdx.x < ncand) {
          const int64_t pos0 = (int64_t)sh.cand[threadIdx.x] * kBlock;
          if (pos0 + kBlock <= nv) {
            const u4* kp = reinterpret_cast<const u4*>(p.tkeys + q * p.tk_stride + pos0);
            const u4 v0 = kp[0], v1 = kp[1];
            ckey[0] = v0[0]; ckey[1] = v0[1]; ckey[2] = v0[2]; ckey[3] = v0[3];
            ckey[4] = v1[0]; ckey[5] = v1[1]; ckey[6] = v1[2]; ckey[7] = v1[3];
          } else {
#pragma unroll
            for (int r = 0; r < kBlock; ++r) ckey[r] = pos0 + r < nv ? p.tkeys[q * p.tk_stride + pos0 + r] : 0u;
          }
          // with at least 512 blocks, the top 512 hold 512 positions whose
          // keys equal their block keys (>= thr), so a position with a key
          // below thr is outranked 512 times: it leaves the candidates
          const uint32_t kfloor = K1 >= (uint32_t)kTopK ? thr : 1u;
#pragma unroll
          for (int r = 0; r < kBlock; ++r) ckey[r] = ckey[r] >= kfloor ? ckey[r] : 0u;
        }
        // With >= 512 blocks at least 512 candidate keys reach the floor (the
        // top 512 blocks' maxima); with fewer, every block is a candidate and
        // every visible position has a nonzero key.  The best block's maximum
        // is the largest key of all.
        c_k2 = K1 >= (uint32_t)kTopK ? (uint32_t)kTopK : (uint32_t)min(nv, (int64_t)kTopK);
        c_kmin = K1 >= (uint32_t)kTopK ? thr : 1u;
        c_kmax = kmax;
      }
      // the pool: for its output (role 0, or role 2 with an output), or for
      // the Top-512 select when the candidates were too many
      if (role == 0 || (role == 2 && p.pool) || ncand < 0) {
        radix_rest<KPT1>(get, st, sh, &sh.hist[0], tau, need);
        compact_topk<KPT1>(get, tau, need, sh, [&](uint32_t o, int j) { sh.pool[o] = (int32_t)(base1 + j); });
      }
    }
  } else if (K1 > 0) {                       // (no visible block: the pool stays empty)
    // More than 16 blocks per thread: rank super-blocks of 8 blocks by their
    // maximum first.  The top 2,048 blocks lie in the top 2,048 super-blocks
    // (ranked by (max desc, id asc)): every super-block ranked above a chosen
    // block's super-block holds a distinct block that outranks that block.
    // Their 16,384 member blocks are then ranked exactly.
    constexpr int SPT = kPoolPositions / kSelThreads;   // 16 super-blocks per thread
    const int64_t nsb = (nb + 7) / 8;
    const int64_t sb0 = (int64_t)threadIdx.x * SPT;
    uint32_t skey[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int64_t b0 = (sb0 + j) * 8;
      uint32_t m = 0u;
      if (b0 + 8 <= nb) {
        const u4* kp = reinterpret_cast<const u4*>(bk + b0);
        const u4 v0 = kp[0], v1 = kp[1];
        m = max(max(max(v0[0], v0[1]), max(v0[2], v0[3])), max(max(v1[0], v1[1]), max(v1[2], v1[3])));
      } else {
        for (int r = 0; r < 8; ++r) m = max(m, b0 + r < nb ? bk[b0 + r] : 0u);
      }
      skey[j] = m;
    }
    hists_clear(sh);
    __syncthreads();
    const uint32_t Ks = (uint32_t)min(nsb, (int64_t)kPoolBlocks);
    {
      auto get = [&](int j) { return skey[j]; };
      uint32_t tau, need, kmin, kmax, cnt;
      key_stats<SPT>(get, sh, kmin, kmax, cnt);
      radix_select<SPT>(get, Ks, kmin, kmax, sh, &sh.hist[0], tau, need);
      compact_topk<SPT>(get, tau, need, sh, [&](uint32_t o, int j) { sh.sbpool[o] = (int32_t)(sb0 + j); });
    }
    for (int i = Ks + threadIdx.x; i < kPoolBlocks; i += kSelThreads) sh.sbpool[i] = -1;
    __syncthreads();
    // member blocks of the chosen super-blocks: thread t takes slots 2t, 2t+1
    uint32_t ckey[2 * 8];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int32_t sb = sh.sbpool[2 * threadIdx.x + jj];
      const int64_t b0 = (int64_t)sb * 8;
      if (sb >= 0 && b0 + 8 <= nb) {
        const u4* kp = reinterpret_cast<const u4*>(bk + b0);
        const u4 v0 = kp[0], v1 = kp[1];
        ckey[8 * jj + 0] = v0[0]; ckey[8 * jj + 1] = v0[1]; ckey[8 * jj + 2] = v0[2]; ckey[8 * jj + 3] = v0[3];
        ckey[8 * jj + 4] = v1[0]; ckey[8 * jj + 5] = v1[1]; ckey[8 * jj + 6] = v1[2]; ckey[8 * jj + 7] = v1[3];
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) ckey[8 * jj + r] = (sb >= 0 && b0 + r < nb) ? bk[b0 + r] : 0u;
      }
    }
    {
      auto get = [&](int j) { return ckey[j]; };
      uint32_t tau, need, kmin, kmax, cnt, thr;
      key_stats<16>(get, sh, kmin, kmax, cnt);
      // the first pass also gives the first digit of the 512th block key:
      // the Top-512 positions lie in the top 512 blocks, whose keys are at
      // least its floor thr (the same argument as the candidates above)
      const RadixState st = radix_first<16>(get, K1, kmin, kmax, sh, &sh.hist[3], min(K1, (uint32_t)kTopK), thr);
      radix_rest<16>(get, st, sh, &sh.hist[3], tau, need);
      const int c0 = threadIdx.x * 16;
      compact_topk<16>(get, tau, need, sh, [&](uint32_t o, int j) {
        const int c = c0 + j;
        sh.pool[o] = sh.sbpool[c >> 3] * 8 + (c & 7);
        sh.pkey[o] = get(j);
      });
      // with fewer than 512 blocks every block counts (pool keys are nonzero)
      if (p.pthr && threadIdx.x == 0) p.pthr[q] = K1 >= (uint32_t)kTopK ? thr : 1u;
    }
    // the position select below needs clean histograms
    __syncthreads();
    {
      u4* hp = reinterpret_cast<u4*>(&sh.hist[3][0]);
      for (int i = threadIdx.x; i < 3 * kDigitBins / 4; i += kSelThreads) hp[i] = u4{0u, 0u, 0u, 0u};
    }
  }
  if (role == 1 && ncand >= 0) {              // ---- Top-512 of the candidates only
    select_positions<kBlock>(ckey, sh, sh.cand, p.topk + q * kTopK, c_k2, c_kmin, c_kmax);
    return;
  }
  for (int i = K1 + threadIdx.x; i < kPoolBlocks; i += kSelThreads) sh.pool[i] = -1;
  __syncthreads();
  if (p.pool && role != 1)
    for (int i = threadIdx.x; i < kPoolBlocks; i += kSelThreads) p.pool[q * kPoolBlocks + i] = sh.pool[i];
  if (p.pkeys && !p.topk) {                  // pool only: its blocks' keys for the rescoring
    for (int i = threadIdx.x; i < kPoolBlocks; i += kSelThreads)
      p.pkeys[q * kPoolBlocks + i] = (uint32_t)i < K1 ? sh.pkey[i] : 0u;
    if (K1 == 0 && threadIdx.x == 0) p.pthr[q] = 1u;
  }
  if (role == 0 || !p.topk) return;

  // ---- step 2: Top-512 positions of the candidate blocks, or of the pool
  if (ncand >= 0) {
    select_positions<kBlock>(ckey, sh, sh.cand, p.topk + q * kTopK, c_k2, c_kmin, c_kmax);
    return;
  }
  uint32_t key[KPT2];
  const int base2 = threadIdx.x * KPT2;
#pragma unroll
  for (int jb = 0; jb < KPT2; jb += kBlock) {           // one pool block = 8 keys, 32 aligned bytes
    const int32_t blk = sh.pool[(base2 + jb) >> 3];
    const int64_t pos0 = (int64_t)blk * kBlock;
    if (blk >= 0 && pos0 + kBlock <= nv) {
      const u4* kp = reinterpret_cast<const u4*>(p.tkeys + q * p.tk_stride + pos0);
      const u4 v0 = kp[0], v1 = kp[1];
      key[jb + 0] = v0[0]; key[jb + 1] = v0[1]; key[jb + 2] = v0[2]; key[jb + 3] = v0[3];
      key[jb + 4] = v1[0]; key[jb + 5] = v1[1]; key[jb + 6] = v1[2]; key[jb + 7] = v1[3];
    } else {
#pragma unroll
      for (int r = 0; r < kBlock; ++r)
        key[jb + r] = (blk >= 0 && pos0 + r < nv) ? p.tkeys[q * p.tk_stride + pos0 + r] : 0u;
    }
  }
  select_positions<KPT2>(key, sh, sh.pool, p.topk + q * kTopK);
}

// ============================================================== reindex
constexpr int kRxSlotsPerWG = 64;
// Score the pool positions of one query: grid (2048 / 64 slots, nq).  A
// workgroup takes 64 pool slots (32 16-token tiles, two blocks each); each of
// its waves loads the block ids of its 8 tiles, then issues all 8 tiles' key
// gathers before the first MFMA, so 16 KiB per wave are in flight at once.
template <int DI, int HI, bool F8>
__global__ __launch_bounds__(256) void k_reindex_score(ReindexParams p) {
  constexpr int KK = DI / 64;
  constexpr int TPW = kRxSlotsPerWG / 2 / 4;        // tiles per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t q = blockIdx.y;
  const int64_t b = q / p.qn;
  int64_t nv = p.nvis ? (int64_t)p.nvis[q] : p.T;
  nv = max((int64_t)0, min(nv, p.T));
  const int64_t nb = (nv + kBlock - 1) / kBlock;

  const int32_t* pool = p.pool + q * kPoolBlocks;
  const int slot0 = blockIdx.x * kRxSlotsPerWG + 2 * TPW * wave + (n >> 3);   // slot of tile u: slot0 + 2u
  int32_t blk[TPW];
  // long Full path: blocks whose Full-layer key lies below the Top-512 floor
  // hold no Top-512 position, and this query is that layer's own, so they
  // are not gathered (their keys stay 0, not candidates)
  uint32_t pk[TPW];
  const uint32_t floor_q = p.pthr ? p.pthr[q] : 0u;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    blk[u] = pool[slot0 + 2 * u];
    pk[u] = p.pkeys ? p.pkeys[q * kPoolBlocks + slot0 + 2 * u] : 0u;
  }

  v4i a[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    v4i z = {0, 0, 0, 0};
    if (n < HI) z = *reinterpret_cast<const v4i*>(p.iq + (q * HI + n) * DI + g * 16 + kk * 64);
    a[kk] = z;
  }
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wv[i] = (4 * g + i < HI) ? p.iw[q * HI + 4 * g + i] : 0.0f;
    if constexpr (F8) wv[i] *= (4 * g + i < HI) ? p.iqs[q * HI + 4 * g + i] : 0.0f;
  }

  const int8_t* ikb = p.ik + b * p.T * DI;
  v4i bf[TPW][KK];
  bool ok[TPW];
  float skv[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t pos = (int64_t)blk[u] * kBlock + (n & 7);
    ok[u] = blk[u] >= 0 && (int64_t)blk[u] < nb && pos < nv && pk[u] >= floor_q;
    skv[u] = 1.0f;
    if constexpr (F8) skv[u] = ok[u] ? p.iks[b * p.T + pos] : 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4i z = {0, 0, 0, 0};
      if (ok[u]) z = *reinterpret_cast<const v4i*>(ikb + pos * DI + g * 16 + kk * 64);
      bf[u][kk] = z;
    }
  }
  uint32_t* ck = p.ckeys + q * kPoolPositions;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    float val[4];
    index_dots<KK, F8>(a, bf[u], val);
#pragma unroll
    for (int i = 0; i < 4; ++i) val[i] *= wv[i];
    float tot;
    if constexpr (HI == 2) {
      tot = val[0] + val[1];
    } else {
      tot = ((val[0] + val[1]) + val[2]) + val[3];
      if constexpr (HI >= 8) tot = sum_swap16(tot);
      if constexpr (HI >= 16) tot = sum_swap32(tot);
    }
    if constexpr (F8) tot *= skv[u];
    const uint32_t key = ok[u] ? score_key(tot) : 0u;
    // the block's maximum: 8 lanes of each half of the 16-lane row
    uint32_t m = key;
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));   // xor 1
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));   // xor 2
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));  // half-row mirror
    if (g == 0) {
      ck[(slot0 + 2 * u) * kBlock + (n & 7)] = key;
      if ((n & 7) == 0) p.bkeys[q * kPoolBlocks + slot0 + 2 * u] = m;
    }
  }
}

// Top-512 of the rescored pool.  As in the Full select, the Top-512 positions
// lie in the top 512 pool blocks (by block maximum, ties to the lower block),
// so the blocks at or above the first radix digit of the 512th block key are
// the candidates; with at least 512 non-empty blocks, a position whose key is
// below that digit's floor is outranked 512 times and leaves too.  When more
// than 1,024 blocks pass, all 16,384 pool positions are selected from.
__global__ __launch_bounds__(kSelThreads) void k_select_reindex(ReindexParams p) {
  constexpr int KPT2 = kPoolPositions / kSelThreads;
  constexpr int BPT = kPoolBlocks / kSelThreads;       // 2 pool slots per thread
  __shared__ SelShared sh;
  const int64_t q = blockIdx.x;
  // the block keys go out first; the histograms are cleared meanwhile
  const u2 bv = *reinterpret_cast<const u2*>(p.bkeys + q * kPoolBlocks + BPT * threadIdx.x);
  const uint32_t bkey[BPT] = {bv[0], bv[1]};
  hists_clear(sh);
  for (int i = threadIdx.x; i < kPoolBlocks; i += kSelThreads) sh.pool[i] = p.pool[q * kPoolBlocks + i];
  __syncthreads();
  auto get = [&](int j) { return bkey[j]; };
  uint32_t kmin, kmax, nblk;
  key_stats<BPT>(get, sh, kmin, kmax, nblk);
  if (nblk > 0) {
    uint32_t unused;
    const uint32_t kx = min(nblk, (uint32_t)kTopK);
    const RadixState st = radix_first<BPT>(get, kx, kmin, kmax, sh, &sh.hist[0], 0u, unused);
    const uint32_t thr = kmin + (st.d1 << st.s1);      // floor of the kx-th block key's first digit
    uint32_t mine = 0, ntot;
#pragma unroll
    for (int j = 0; j < BPT; ++j) mine += bkey[j] >= thr ? 1u : 0u;
    uint32_t o = block_excl_scan_total(mine, sh, ntot);
    if (ntot <= (uint32_t)kSelThreads) {
#pragma unroll
      for (int j = 0; j < BPT; ++j)
        if (bkey[j] >= thr) {
          sh.cand[o] = BPT * (int)threadIdx.x + j;        // pool slot
          sh.sbpool[o] = sh.pool[BPT * threadIdx.x + j];  // its block id
          ++o;
        }
      __syncthreads();
      uint32_t ckey[kBlock] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      if (threadIdx.x < ntot) {
        const u4* kp = reinterpret_cast<const u4*>(p.ckeys + q * kPoolPositions + (int64_t)sh.cand[threadIdx.x] * kBlock);
        const u4 v0 = kp[0], v1 = kp[1];
        const uint32_t kfloor = nblk >= (uint32_t)kTopK ? thr : 1u;
        ckey[0] = v0[0]; ckey[1] = v0[1]; ckey[2] = v0[2]; ckey[3] = v0[3];
        ckey[4] = v1[0]; ckey[5] = v1[1]; ckey[6] = v1[2]; ckey[7] = v1[3];
#pragma unroll
        for (int r = 0; r < kBlock; ++r) ckey[r] = ckey[r] >= kfloor ? ckey[r] : 0u;
      }
      select_positions<kBlock>(ckey, sh, sh.sbpool, p.topk + q * kTopK);
      return;
    }
  }
  uint32_t key[KPT2];
  const int base = threadIdx.x * KPT2;
#pragma unroll
  for (int j = 0; j < KPT2; ++j) key[j] = p.ckeys[q * kPoolPositions + base + j];
  select_positions<KPT2>(key, sh, sh.pool, p.topk + q * kTopK);
}

// ============================================================== launchers
hipError_t launch_select_full(const SelectParams& p, int nq, int64_t max_blocks, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  SelectParams pp = p;
  // with a pool output, the pool and the Top-512 take one workgroup each (up
  // to 8,192 blocks); a small quantisation job rides along as extra
  // workgroups (four lanes per 16-channel group), a larger one is launched
  // first on its own
  if (max_blocks > 128 * kSelThreads) return hipErrorInvalidValue;
  // the pool alone (no Top-512) is selected only for the super-block path
  if (!p.topk && (max_blocks <= 8 * kSelThreads || !p.pool)) return hipErrorInvalidValue;
  pp.roles = (max_blocks <= 8 * kSelThreads && p.pool) ? 2 : 1;
  pp.sel_wgs = pp.roles * nq;
  int extra = 0;
  if (p.qj.rows > 0) {
    if (quantize_fits_quad(p.qj.rows, 16 * p.qj.groups)) {
      extra = (int)((4 * p.qj.rows * p.qj.groups + kSelThreads - 1) / kSelThreads);
    } else {
      const hipError_t e = p.qj.pg.bt
          ? launch_quantize_paged(p.qj.x, p.qj.xs, p.qj.rows, 16 * p.qj.groups, p.qj.pg, p.qj.codes, p.qj.cs,
                                  p.qj.scales, p.qj.ss, st)
          : launch_quantize(p.qj.x, p.qj.xs, p.qj.rows, 16 * p.qj.groups, p.qj.codes, p.qj.cs, p.qj.scales,
                            p.qj.ss, st);
      if (e != hipSuccess) return e;
    }
  }
  const dim3 grid((unsigned)(pp.sel_wgs + extra));
  if (max_blocks <= 8 * kSelThreads)
    hipLaunchKernelGGL((k_select_full<8>), grid, dim3(kSelThreads), 0, st, pp);
  else if (max_blocks <= 128 * kSelThreads)
    hipLaunchKernelGGL((k_select_full<128>), grid, dim3(kSelThreads), 0, st, pp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_reindex(const ReindexParams& p, int nq, int heads, int dim, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  const dim3 grid(kPoolBlocks / kRxSlotsPerWG, nq);
#define CSA2_RX_CASE(D, H)                                                              \
  if (dim == D && heads == H) {                                                         \
    if (p.iks) hipLaunchKernelGGL((k_reindex_score<D, H, true>), grid, dim3(256), 0, st, p); \
    else hipLaunchKernelGGL((k_reindex_score<D, H, false>), grid, dim3(256), 0, st, p);    \
  } else
  CSA2_RX_CASE(64, 2) CSA2_RX_CASE(64, 4) CSA2_RX_CASE(64, 8) CSA2_RX_CASE(64, 16)
  CSA2_RX_CASE(128, 2) CSA2_RX_CASE(128, 4) CSA2_RX_CASE(128, 8) CSA2_RX_CASE(128, 16)
  { return hipErrorInvalidValue; }
#undef CSA2_RX_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_reindex, dim3(nq), dim3(kSelThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace csa2
