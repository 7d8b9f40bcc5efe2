// Device-side check of the indexer's rows against their contract (the
// pool and Top-K rows that the Full and Reindex calls write, and the shape
// of the pool a Reindex call is given).
//
// The contract follows the DeepSeek-V4.1-Flash pages (ai-maestro.online,
// "Compressed Sparse Attention 2": a pool of 2,048 eight-token blocks, a
// fresh Top-512 taken from it; Reindex rescores the pool of the Full layer
// for the same query tokens) in the canonical form the library writes:
// ascending ids, -1 only as trailing padding.
#include "check.h"

namespace csa2 {

namespace {
constexpr int kChkThreads = 256;

// number of rows flagged by the workgroup (thread 0 adds 1 per bad row)
CSA2_DEV void flag_row(bool bad, int* sh_bad) {
  if (bad) atomicOr(sh_bad, 1);
}
}  // namespace

// One workgroup per query.  mode 0: Full outputs (pool may be absent);
// 1: Reindex outputs (topk against the given pool); 2: the shape of a
// Reindex input pool only.
__global__ __launch_bounds__(kChkThreads) void k_check_index(CheckParams p) {
  __shared__ int32_t pool[kPoolBlocks];
  __shared__ int sh_pool_bad, sh_topk_bad;
  __shared__ uint32_t sh_pc, sh_tc, sh_npos;
  const int64_t q = blockIdx.x;
  int64_t nv = p.nvis ? (int64_t)p.nvis[q] : p.T;
  nv = max((int64_t)0, min(nv, p.T));
  const int64_t nb = (nv + kBlock - 1) / kBlock;
  if (threadIdx.x == 0) { sh_pool_bad = 0; sh_topk_bad = 0; sh_pc = 0; sh_tc = 0; sh_npos = 0; }
  const bool has_pool = p.pool != nullptr;
  if (has_pool)
    for (int i = threadIdx.x; i < kPoolBlocks; i += kChkThreads) pool[i] = p.pool[q * kPoolBlocks + i];
  __syncthreads();

  // ---- pool: leading ids >= 0, strictly ascending, then -1 only; a Full
  // pool's ids lie in [0, nb) and number min(2048, nb)
  if (has_pool) {
    uint32_t pc = 0, npos = 0;
    bool bad = false;
    for (int i = threadIdx.x; i < kPoolBlocks; i += kChkThreads) {
      const int32_t v = pool[i];
      if (v >= 0) {
        ++pc;
        if (i > 0 && !(pool[i - 1] >= 0 && pool[i - 1] < v)) bad = true;
        if (p.mode == 0 && (int64_t)v >= nb) bad = true;
        if ((int64_t)v < nb) npos += (uint32_t)min((int64_t)kBlock, nv - (int64_t)v * kBlock);
      } else if (v != -1) {
        bad = true;
      }
    }
    flag_row(bad, &sh_pool_bad);
    atomicAdd(&sh_pc, pc);
    atomicAdd(&sh_npos, npos);
  }
  __syncthreads();
  if (has_pool && p.mode == 0 && threadIdx.x == 0 && (int64_t)sh_pc != min(nb, (int64_t)kPoolBlocks)) sh_pool_bad = 1;

  // ---- Top-K: leading positions >= 0, strictly ascending, each in [0, nv)
  // and inside a pool block (when a pool is given), then -1 only; the count
  // is min(512, nv) for a Full row, min(512, positions of the pool) for a
  // Reindex row
  if (p.mode != 2) {
    const int32_t* tk = p.topk + q * kTopK;
    uint32_t tc = 0;
    bool bad = false;
    const int pcount = (int)sh_pc;
    for (int i = threadIdx.x; i < kTopK; i += kChkThreads) {
      const int32_t v = tk[i];
      if (v >= 0) {
        ++tc;
        if (i > 0 && !(tk[i - 1] >= 0 && tk[i - 1] < v)) bad = true;
        if ((int64_t)v >= nv) bad = true;
        if (has_pool) {                          // binary search of block v / 8 in the ascending pool prefix
          const int32_t blk = v >> 3;
          int lo = 0, hi = pcount;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (pool[mid] < blk) lo = mid + 1;
            else hi = mid;
          }
          if (lo >= pcount || pool[lo] != blk) bad = true;
        }
      } else if (v != -1) {
        bad = true;
      }
    }
    flag_row(bad, &sh_topk_bad);
    atomicAdd(&sh_tc, tc);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int topk_bad = sh_topk_bad;
    if (p.mode == 0 && (int64_t)sh_tc != min(nv, (int64_t)kTopK)) topk_bad = 1;
    if (p.mode == 1 && has_pool && sh_tc != min(sh_npos, (uint32_t)kTopK)) topk_bad = 1;
    const uint32_t n_bad = (uint32_t)(sh_pool_bad != 0) + (uint32_t)(p.mode != 2 && topk_bad != 0);
    if (n_bad) atomicAdd(p.bad, n_bad);
  }
}

hipError_t launch_check_index(const CheckParams& p, int nq, hipStream_t st) {
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_check_index, dim3(nq), dim3(kChkThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace csa2
