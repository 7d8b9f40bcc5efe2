// FP4 (E2M1 codes, one E4M3 scale per 16 channels) quantise / dequantise of
// main-KV rows for gfx950.
//
// Method: DeepSeek-V4.1-Flash pages, ai-maestro.online section "FP4 KV,
// Bounded Replay, and other extensions": the main KV quantises to E2M1 with
// one E4M3 scale per 16 channels, NVFP4 without its global scale.  The scale
// of a group is E4M3(amax / 6) and each element is E2M1(x / scale), both
// rounded to nearest with ties to the even code and saturating (448 and 6).
//
// Exactness: neither quotient is ever formed.  Rounding y = amax/6 to the
// E4M3 grid only needs the sign of amax - 6*mu for midpoints mu between
// neighbouring grid values, and 6*mu (<= 7 significant bits) is exact in
// fp32; likewise |x| / s against the E2M1 midpoints 0.25 .. 5 compares
// |x| with m*s, exact in fp32 (<= 7 significant bits).  So every decision is
// the exact-arithmetic one.
//
// A decode step quantises B new rows (latency-bound): four lanes take one
// 16-channel group there, 16 B of fp32 in and 2 code bytes out each.  Bulk
// quantisation of a cache (a one-off) takes one thread per group.
#include "quant_dev.h"
#include "quant.h"

namespace csa2 {

// T: float (fp32 rows) or uint16_t (bf16 rows, widened exactly to fp32)
template <class T>
__global__ __launch_bounds__(256) void k_quantize_group(const T* __restrict__ x, int64_t xs, int64_t rows,
                                                  int groups, uint8_t* __restrict__ codes, int64_t cs,
                                                  uint8_t* __restrict__ scales, int64_t ss) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * groups) return;
  const int64_t r = gid / groups;
  const int g = (int)(gid - r * groups);
  const T* src = x + r * xs + 16 * g;
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[4];
    load4(src + 4 * i, f);
    v[4 * i] = f[0]; v[4 * i + 1] = f[1]; v[4 * i + 2] = f[2]; v[4 * i + 3] = f[3];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = scale_code(amax);
  const float s = e4m3_pos(sc);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = (s == 0.0f) ? ((__float_as_uint(v[i]) >> 28) & 8u) : element_code(v[i], s);
    if (i < 8) lo |= c << (4 * i); else hi |= c << (4 * (i - 8));
  }
  *reinterpret_cast<u2*>(codes + r * cs + 8 * g) = u2{lo, hi};
  scales[r * ss + g] = (uint8_t)sc;
}


// Four lanes per 16-channel group, four channels each (small launches such
// as a decode step's new rows, where latency rules): coalesced 16-byte loads,
// the group's amax over the lane quad by DPP (max is exact and ignores NaN in
// any order), then each lane writes its 4 codes (2 bytes) and the quad's
// first lane the scale.
template <class T>
__global__ __launch_bounds__(256) void k_quantize_quad(const T* __restrict__ x, int64_t xs, int64_t rows,
                                                  int groups, uint8_t* __restrict__ codes, int64_t cs,
                                                  uint8_t* __restrict__ scales, int64_t ss) {
  quantize_quad_thread(x, xs, rows, groups, codes, cs, scales, ss, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// New rows into a paged cache: row r goes to position pos[r] of sequence
// seq[r], i.e. cache row block_table[seq][pos / P] * P + pos % P.  Rows whose
// sequence, position or page is out of range are skipped.
__global__ __launch_bounds__(256) void k_quantize_paged(const float* __restrict__ x, int64_t xs, int64_t rows,
                                                   int groups, uint8_t* __restrict__ codes, int64_t cs,
                                                   uint8_t* __restrict__ scales, int64_t ss, PagedRows d) {
  quantize_quad_thread_to(x, xs, rows, groups, codes, cs, scales, ss, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                          [&](int64_t r) { return paged_row(d, r); });
}

hipError_t launch_quantize_paged(const float* x, int64_t xs, int64_t rows, int dim, const PagedRows& d,
                                 uint8_t* codes, int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st) {
  const int groups = dim / 16;
  const int64_t n = rows * groups;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_paged, dim3((unsigned)((4 * n + 255) / 256)), dim3(256), 0, st, x, xs, rows, groups,
                     codes, cs, scales, ss, d);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes, int64_t cs,
                                                    const uint8_t* __restrict__ scales, int64_t ss,
                                                    int64_t rows, int groups, float* __restrict__ out,
                                                    int64_t os) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * groups) return;
  const int64_t r = gid / groups;
  const int g = (int)(gid - r * groups);
  const u2 c = *reinterpret_cast<const u2*>(codes + r * cs + 8 * g);
  const _Float16 s = e4m3_to_half<0>(scales[r * ss + g]);
  const v8h a = fp4x8_to_half(c[0], s);
  const v8h b = fp4x8_to_half(c[1], s);
  float4* dst = reinterpret_cast<float4*>(out + r * os + 16 * g);
  dst[0] = make_float4((float)a[0], (float)a[1], (float)a[2], (float)a[3]);
  dst[1] = make_float4((float)a[4], (float)a[5], (float)a[6], (float)a[7]);
  dst[2] = make_float4((float)b[0], (float)b[1], (float)b[2], (float)b[3]);
  dst[3] = make_float4((float)b[4], (float)b[5], (float)b[6], (float)b[7]);
}

bool quantize_fits_quad(int64_t rows, int dim) { return rows * (dim / 16) <= kQuantQuadMaxGroups; }

template <class T>
static hipError_t launch_quantize_t(const T* x, int64_t xs, int64_t rows, int dim, uint8_t* codes,
                                    int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st) {
  const int groups = dim / 16;
  const int64_t n = rows * groups;
  if (n == 0) return hipSuccess;
  if (n <= kQuantQuadMaxGroups) {                 // four lanes per group
    hipLaunchKernelGGL(k_quantize_quad<T>, dim3((unsigned)((4 * n + 255) / 256)), dim3(256), 0, st, x, xs, rows,
                       groups, codes, cs, scales, ss);
  } else {
    hipLaunchKernelGGL(k_quantize_group<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, xs, rows,
                       groups, codes, cs, scales, ss);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t xs, int64_t rows, int dim, uint8_t* codes,
                           int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st) {
  return launch_quantize_t(x, xs, rows, dim, codes, cs, scales, ss, st);
}

hipError_t launch_quantize_bf16(const uint16_t* x, int64_t xs, int64_t rows, int dim, uint8_t* codes,
                                int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st) {
  return launch_quantize_t(x, xs, rows, dim, codes, cs, scales, ss, st);
}

// ---------------------------------------------------------------- 8-bit window rows
// One wave per bf16 row of `dim` <= 512 channels, 8 channels per lane (the
// encoding is swa8_encode_row in quant_dev.h).
__global__ __launch_bounds__(256) void k_quantize_swa8(const uint16_t* __restrict__ x, int64_t xs, int64_t rows,
                                                       int dim, uint8_t* __restrict__ out, int64_t os,
                                                       float* __restrict__ scales, int64_t ss) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;                         // whole waves
  const bool act = lane < dim / 8;
  const u4 w = act ? *reinterpret_cast<const u4*>(x + row * xs + 8 * lane) : u4{0u, 0u, 0u, 0u};
  float sc;
  const u2 c = swa8_encode_row(w, sc);
  if (act) *reinterpret_cast<u2*>(out + row * os + 8 * lane) = c;
  if (lane == 0) scales[row * ss] = sc;
}

hipError_t launch_quantize_swa8(const uint16_t* x, int64_t xs, int64_t rows, int dim, uint8_t* out, int64_t os,
                                float* scales, int64_t ss, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_swa8, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, x, xs, rows, dim, out, os,
                     scales, ss);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, int64_t cs, const uint8_t* scales, int64_t ss,
                             int64_t rows, int dim, float* out, int64_t os, hipStream_t st) {
  const int groups = dim / 16;
  const int64_t n = rows * groups;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)blocks), dim3(256), 0, st, codes, cs, scales, ss, rows,
                     groups, out, os);
  return hipGetLastError();
}

}  // namespace csa2
