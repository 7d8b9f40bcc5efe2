// Full-layer indexer scan of CSA2 for gfx950: a score for every visible
// position of every query, plus the 8-token block maxima.
//
// Method: DeepSeek-V4.1-Flash pages, ai-maestro.online section "Compressed
// Sparse Attention 2": a Full layer scores the whole context with its
// indexer; its hierarchical indexer keeps a pool of blocks of eight tokens.
// Score s(q,t) = sum_h w[q,h] * relu(q_h . k_t); block score = max over its
// visible tokens.  The selection that follows is in select.hip.  The pages
// leave the indexer's precision open: int8 keys and queries (exact integer
// dot products), or E4M3FN codes with one fp32 scale per key position and
// per (query, head), scored as sk[t] * sum_h (w[q,h] * sq[q,h]) *
// relu(E4M3 dot product) (equal to the dequantised score for positive
// scales).
//
// Design (gfx950, wave64): the indexer keys stream once from HBM.  Each wave
// takes 16-token tiles: an int8 MFMA 16x16x64 contracts the 16 token rows (B
// operand, one token per lane column) with up to 64 score rows (A operand: 64
// of the sequence's Qn * H_I query-head rows, 32 for E4M3 operands; more rows
// take more workgroups, so prefill chunks reuse the keys from L2), so the dot
// products are exact int32.  ReLU, head weights and the head sum run on the 4 accumulator rows a
// lane holds plus cross-lane adds; the 8-token block maximum is three DPP max
// steps inside each 16-lane row.  Token keys and block keys (order-preserving
// uint32 of the fp32 score) go to the workspace.
#include "common.h"

namespace csa2 {

// Channel order of the int8 operands: lane group g takes, in k-step kk, the 16
// channels 16g + 64kk .. +15, so the 4 lanes of a key row read 64 contiguous
// bytes per load (the contraction only needs both operands to agree).
// HI: indexer heads (2, 4, 8, 16); DI: indexer dim (64, 128); F8: E4M3 codes;
// MTX: M tiles (16 score rows each) per workgroup.  Fewer M tiles hold fewer
// query operands in registers (more waves per SIMD); more M tiles read each
// key tile for more score rows.  NT: the keys are read by one workgroup per
// key tile (non-temporal loads).
template <int DI, int HI, bool F8, int MTX, bool NT>
__global__ __launch_bounds__(256) void k_index_scan(ScanParams p) {
  constexpr int KK = DI / 64;                 // MFMAs per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  // score rows (query j, head h) -> row j*HI + h; this workgroup takes rows
  // [r0, r0 + rows_used) of its sequence, at most 16 * MTX
  const int r0 = 16 * MTX * (int)blockIdx.z;
  const int rows_used = min(16 * MTX, p.qn * HI - r0);
  const int MT = (rows_used + 15) >> 4;
  const int j_lo = r0 / HI, j_hi = (r0 + rows_used - 1) / HI;

  // furthest visible position over the workgroup's queries
  int64_t vmax = p.T;
  if (p.nvis) {
    vmax = 0;
    for (int j = j_lo; j <= j_hi; ++j) vmax = max(vmax, (int64_t)p.nvis[b * p.qn + j]);
    vmax = min(vmax, p.T);
  }
  const int64_t t0 = 0, tend = vmax;

  // A operands (score rows) and weights of the 4 output rows each lane holds
  v4i a[MTX][KK];
  float wv[MTX][4];
#pragma unroll
  for (int mt = 0; mt < MTX; ++mt) {
    const int r = 16 * mt + n;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4i z = {0, 0, 0, 0};
      if (mt < MT && r < rows_used) {
        const int j = (r0 + r) / HI, h = (r0 + r) % HI;
        z = *reinterpret_cast<const v4i*>(p.iq + ((int64_t)(b * p.qn + j) * HI + h) * DI + g * 16 + kk * 64);
      }
      a[mt][kk] = z;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r2 = 16 * mt + 4 * g + i;
      float w = 0.0f;
      if (mt < MT && r2 < rows_used) {
        const int64_t wi = (int64_t)(b * p.qn + (r0 + r2) / HI) * HI + (r0 + r2) % HI;
        w = p.iw[wi];
        if constexpr (F8) w *= p.iqs[wi];
      }
      wv[mt][i] = w;
    }
  }
  int nvq[MTX];   // visibility of the queries whose rows this lane's group holds (HI >= 4 case)
#pragma unroll
  for (int mt = 0; mt < MTX; ++mt) {
    const int j = (r0 + 16 * mt + 4 * g) / HI;
    nvq[mt] = (int)min((int64_t)(p.nvis && j < p.qn ? p.nvis[b * p.qn + j] : p.T), p.T);
  }

  const int8_t* ikb = p.ik + (int64_t)b * p.T * DI;
  const float* iksb = F8 ? p.iks + (int64_t)b * p.T : nullptr;
  const int ntile = (int)((tend - t0 + 15) >> 4);

  // score one 16-token tile whose indexer-key fragments are in bf (sk: the
  // FP8 key scale of this lane's token)
  auto process = [&](int it, const v4i (&bf)[KK], float sk) {
    const int64_t t = t0 + 16 * it + n;
    const bool tok_ok = t < tend;
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt) {
      if (mt >= MT) break;
      float val[4];
      index_dots<KK, F8>(a[mt], bf, val);
#pragma unroll
      for (int i = 0; i < 4; ++i) val[i] *= wv[mt][i];
      if constexpr (HI >= 4) {
        float tot = ((val[0] + val[1]) + val[2]) + val[3];
        if constexpr (HI >= 8) tot = sum_swap16(tot);
        if constexpr (HI >= 16) tot = sum_swap32(tot);
        if constexpr (F8) tot *= sk;
        const int j = (r0 + 16 * mt + 4 * g) / HI;   // query within the sequence
        const uint32_t key = (tok_ok && t < nvq[mt] && j < p.qn) ? score_key(tot) : 0u;
        // 8-token block max inside each half of the 16-lane row
        uint32_t m = key;
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // xor 1
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));  // xor 2
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false)); // half-row mirror
        const bool writer = (HI == 4) || (HI == 8 && (g & 1) == 0) || (HI == 16 && g == 0);
        if (writer && j < p.qn && tok_ok) {
          const int64_t q = (int64_t)b * p.qn + j;
          if (p.tkeys) p.tkeys[q * p.tk_stride + t] = key;      // NULL: block maxima only
          if ((n & 7) == 0) p.bkeys[q * p.bk_stride + (t >> 3)] = m;
        }
      } else {  // HI == 2: rows (i0,i1) and (i2,i3) are two queries
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
          float tot = val[2 * hq] + val[2 * hq + 1];
          if constexpr (F8) tot *= sk;
          const int j = (r0 + 16 * mt + 4 * g) / 2 + hq;
          const int nv = (int)min((int64_t)(p.nvis && j < p.qn ? p.nvis[b * p.qn + j] : p.T), p.T);
          const uint32_t key = (tok_ok && t < nv && j < p.qn) ? score_key(tot) : 0u;
          uint32_t m = key;
          m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
          m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
          m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
          if (j < p.qn && tok_ok) {
            const int64_t q = (int64_t)b * p.qn + j;
            if (p.tkeys) p.tkeys[q * p.tk_stride + t] = key;
            if ((n & 7) == 0) p.bkeys[q * p.bk_stride + (t >> 3)] = m;
          }
        }
      }
    }
  };

  // The workgroups of a sequence sweep its keys together: in each round they
  // take 16 consecutive tiles each out of one contiguous stretch of
  // 16 * gridDim.x tiles, so the requests in flight across the GPU stay close
  // in memory.  Wave w takes tiles 4u + w of its workgroup's 16.
  //
  // The keys go straight to LDS (global_load_lds_dwordx4): each instruction
  // reads 1 KiB of whole key rows, lane l taking 16 bytes, and lands them in
  // the wave's tile buffer in lane order.  A row-dependent XOR swizzle of the
  // 16-byte chunk each lane fetches (chunk p of row r holds key chunk
  // p ^ swz(r)) makes the operand reads below, row n and chunk g + 4kk per
  // lane, hit 16 distinct bank groups per 16 lanes.  All U tiles are issued
  // before the first MFMA.
  constexpr int U = 4;
  // With one score-row group per sequence (decode, verify) the keys are read
  // once per step and never again within it: non-temporal loads (cache
  // policy NT) stream them past the last-level cache, so the step's other
  // working set (the attention's window rows and gathered FP4 rows, which
  // decode re-reads from one step to the next) stays resident.  With several
  // groups (prefill) every group reads each key tile, and the later reads
  // should hit the cache: normal policy.
  constexpr int kNonTemporal = NT ? 2 : 0;
  constexpr int CPR = DI / 16;                 // 16-byte chunks per key row
  constexpr int RPI = 1024 / DI;               // rows per 1 KiB load instruction
  constexpr int NI = 16 * DI / 1024;           // load instructions per 16-row tile
  constexpr int SWD = 16 / CPR;                // swz(r) = (r / SWD) % CPR
  __shared__ __attribute__((aligned(16))) int8_t kbuf[4][U][16 * DI];
  int8_t* const mybuf = &kbuf[wave][0][0];
  for (int64_t base = 16 * (int64_t)blockIdx.x; base < ntile; base += 16 * (int64_t)gridDim.x) {
    float skv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      skv[u] = 1.0f;
      if constexpr (F8) {
        const int64_t t = 16 * (base + 4 * u + wave) + n;
        if (t < tend) skv[u] = NT ? __builtin_nontemporal_load(iksb + t) : iksb[t];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ ((r / SWD) % CPR);
        const int64_t t = 16 * (base + 4 * u + wave) + r;
        const int64_t row = t < tend ? t : 0;
        __builtin_amdgcn_global_load_lds(ikb + row * DI + c * 16,
                                         (__attribute__((address_space(3))) void*)(mybuf + u * 16 * DI + i * 1024),
                                         16, 0, kNonTemporal);
      }
    }
    // s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maximum): the tiles
    // are in this wave's LDS buffer; the compiler does not order LDS-bound
    // loads before the reads below by itself
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i bf[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        bf[kk] = *reinterpret_cast<const v4i*>(mybuf + u * 16 * DI + n * DI + ((g + 4 * kk) ^ ((n / SWD) % CPR)) * 16);
      if (base + 4 * u + wave < ntile) process((int)(base + 4 * u + wave), bf, skv[u]);
    }
  }
}

// ============================================================== launcher
template <int DI, int HI>
static void launch_scan_t(const ScanParams& p, hipStream_t st) {
  // two M tiles for E4M3 operands (whose fp16 decodes the compiler keeps for
  // the whole loop) and for sequences of at most 32 score rows (decode: 84
  // instead of 118 VGPRs, 5 waves per SIMD); four otherwise
  const bool two = p.iks || (int64_t)p.qn * HI <= 32;
  const int rows = two ? 32 : 64;                            // score rows per workgroup
  const int64_t groups = ((int64_t)p.qn * HI + rows - 1) / rows;
  // Tokens per workgroup.  The int8 decode scan: 256, one round of 16 tiles
  // (batch-32, 64K-entry decode group: step 122 us against 123 / 124.5 /
  // 126 us with 512 / 1024 / 128).  Every other instantiation: 1024, where
  // 256 was slower (E4M3 decode scan 53.2 vs 49.2 us, prefill 0.88 vs
  // 0.64 ms, 1M-entry verify 268 vs 260 us).
  const int64_t chunk = (!p.iks && two) ? 256 : 1024;
  const int64_t chunks = (p.T + chunk - 1) / chunk;
  const dim3 grid((unsigned)chunks, (unsigned)p.batch, (unsigned)groups);
  const bool once = groups == 1;                             // each key tile read by one workgroup
  if (p.iks) {
    if (once) hipLaunchKernelGGL((k_index_scan<DI, HI, true, 2, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_index_scan<DI, HI, true, 2, false>), grid, dim3(256), 0, st, p);
  } else if (two) {                                          // groups == 1
    hipLaunchKernelGGL((k_index_scan<DI, HI, false, 2, true>), grid, dim3(256), 0, st, p);
  } else {
    if (once) hipLaunchKernelGGL((k_index_scan<DI, HI, false, 4, true>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((k_index_scan<DI, HI, false, 4, false>), grid, dim3(256), 0, st, p);
  }
}

hipError_t launch_index_scan(const ScanParams& p, int heads, int dim, hipStream_t st) {
  if (p.T == 0 || p.batch == 0) return hipSuccess;
#define CSA2_SCAN_CASE(D, H) if (dim == D && heads == H) { launch_scan_t<D, H>(p, st); return hipGetLastError(); }
  CSA2_SCAN_CASE(64, 2) CSA2_SCAN_CASE(64, 4) CSA2_SCAN_CASE(64, 8) CSA2_SCAN_CASE(64, 16)
  CSA2_SCAN_CASE(128, 2) CSA2_SCAN_CASE(128, 4) CSA2_SCAN_CASE(128, 8) CSA2_SCAN_CASE(128, 16)
#undef CSA2_SCAN_CASE
  return hipErrorInvalidValue;
}

}  // namespace csa2
