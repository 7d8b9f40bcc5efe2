// Achievable HBM read rate of the device: every byte of a buffer read once
// with 16-byte non-temporal loads, no arithmetic beyond an XOR that keeps the
// loads live.  Not a step of the method: a reference point for the fraction
// of the 8 TB/s peak that the streaming kernels reach.  Each workgroup reads
// one contiguous chunk (64 KiB of a 1 GiB buffer with 16,384 workgroups):
// on one MI355X 6.75-6.89 TB/s, against 6.0-6.3 TB/s for a grid-stride
// sweep of the same buffer (2,048-16,384 workgroups, 1-8 loads in flight
// per thread).
#include "rate.h"

namespace csa2 {

namespace {
constexpr int kRateThreads = 256;
constexpr int kRateUnroll = 4;                   // 16-byte loads in flight per thread per round
}  // namespace

__global__ __launch_bounds__(kRateThreads) void k_read_rate(const u4* __restrict__ buf, int64_t n16,
                                                            uint32_t* __restrict__ sink) {
  const int64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n16 ? lo + chunk : n16;
  uint32_t x = 0u;
  int64_t i = lo + threadIdx.x;
  for (; i + (kRateUnroll - 1) * kRateThreads < hi; i += kRateUnroll * kRateThreads) {
    u4 v[kRateUnroll];
#pragma unroll
    for (int u = 0; u < kRateUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kRateThreads);
#pragma unroll
    for (int u = 0; u < kRateUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += kRateThreads) {
    const u4 v = __builtin_nontemporal_load(buf + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one word per wave (the lanes' XOR), so the loads cannot be dropped
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (kRateThreads / 64) + (threadIdx.x >> 6)] = x;
}

hipError_t launch_read_rate(const void* buf, int64_t bytes, uint32_t* sink, int wgs, hipStream_t st) {
  if (bytes < 16) return hipSuccess;
  hipLaunchKernelGGL(k_read_rate, dim3((unsigned)wgs), dim3(kRateThreads), 0, st, static_cast<const u4*>(buf),
                     bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace csa2
