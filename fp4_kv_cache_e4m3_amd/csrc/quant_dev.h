// Device-side FP4 (E2M1 + E4M3 per 16 channels) quantisation of main-KV rows,
// shared by the quantise kernels and the fused Full-selection launch.
// Method and exactness argument: see quant.hip's header (DeepSeek-V4.1-Flash
// pages, ai-maestro.online, "FP4 KV, Bounded Replay, and other extensions").
#pragma once

#include "common.h"

namespace csa2 {

// ---------------------------------------------------------------- 8-bit window rows
// A window row is stored as E4M3 codes with one power-of-two scale 2^k per
// row: k is the smallest integer with max|x| <= 448 * 2^k (0 for an all-zero
// row), and each |x| / 2^k (exact) is rounded to the nearest E4M3 value, ties
// to even, with the sign bit of x.  The rounding is exact: on the subnormal
// grid y * 512 is an integer grid coordinate, on a binade y * 2^(3-e) lies in
// [8, 16); both are exact scalings, and v_rndne_f32 rounds them half-even.
CSA2_DEV uint32_t e4m3_rne_code(float y) {          // 0 <= y <= 448
  if (y < 0x1p-6f) return (uint32_t)__builtin_rintf(y * 512.0f);      // codes 0..8 (8 = 2^-6)
  int E;
  (void)__builtin_frexpf(y, &E);                  // y = f * 2^E, f in [0.5, 1)
  const int m = (int)__builtin_rintf(__builtin_ldexpf(y, 4 - E));     // 8 .. 16
  return (uint32_t)((E + 6) * 8 + m - 8);
}

// One row spread over a wave, eight bf16 channels per lane (w, channel order;
// lanes past the row hold zeros): the lane's eight E4M3 codes as two words,
// and the row scale 2^k in sc (every lane).
CSA2_DEV u2 swa8_encode_row(u4 w, float& sc) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  int k = 0;
  if (amax > 0.0f) {
    int e;
    const float f = __builtin_frexpf(amax, &e);    // amax = f * 2^e; 448 = 0.875 * 2^9
    k = e - 9 + (f > 0.875f ? 1 : 0);
  }
  uint32_t word[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = e4m3_rne_code(__builtin_ldexpf(fabsf(v[i]), -k)) | ((__float_as_uint(v[i]) >> 24) & 0x80u);
    word[i / 4] |= c << (8 * (i % 4));
  }
  sc = __builtin_ldexpf(1.0f, k);
  return u2{word[0], word[1]};
}

// launches of at most this many 16-channel groups use four lanes per group
constexpr int64_t kQuantQuadMaxGroups = 8192;

// value of non-negative finite E4M3 code c (0..126) as fp32 (exact)
CSA2_DEV float e4m3_pos(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
}

// E4M3 code of amax/6: nearest, ties to even, saturating at 448 (0x7E).
// The code is n = #{c in 0..125 : 6 * mu_c < amax} for the midpoints mu_c
// between grid values c and c + 1, raised to the even neighbour on a tie.
// An fp32 estimate y' of amax/6 (relative error ~2^-23, against a grid
// spacing of at least 1/16) has grid floor ce within one code of the true
// floor f, and n is f or f + 1; so every c <= ce - 2 counts, every
// c >= ce + 2 does not, and only mu_{ce-2} .. mu_{ce+1} are compared, each
// exactly (6 * mu is exact in fp32).
CSA2_DEV uint32_t scale_code(float amax) {
  const float yp = amax * (1.0f / 6.0f);
  int ce;
  if (!(yp < 448.0f)) ce = 126;
  else if (yp < 0x1p-6f) ce = (int)(yp * 512.0f);                // subnormal grid, step 2^-9
  else ce = ((int)((__float_as_uint(yp) >> 23) & 0xFFu) - 120) * 8 + (int)((__float_as_uint(yp) >> 20) & 7u);
  const int base = ce - 2;
  int n = base;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = base + k;
    const bool below = c < 0 ? true
                     : c > 125 ? false
                               : 3.0f * (e4m3_pos((uint32_t)c) + e4m3_pos((uint32_t)c + 1)) < amax;   // 6 * mu_c, exact
    n += below ? 1 : 0;
  }
  uint32_t c = (uint32_t)n;
  if (c < 126u) {
    const float t = 3.0f * (e4m3_pos(c) + e4m3_pos(c + 1));
    if (t == amax && (c & 1u)) c += 1;                             // tie -> even code
  }
  return c;
}

// E2M1 code of x / s for s > 0: nearest, ties to even, saturating at 6.
CSA2_DEV uint32_t element_code(float x, float s) {
  const float a = fabsf(x);
  const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t cnt = 0;
  bool tie = false;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float t = mids[j] * s;                                   // exact
    cnt += (t < a) ? 1u : 0u;
    tie |= (t == a);
  }
  const uint32_t mag = cnt + ((tie && (cnt & 1u)) ? 1u : 0u);
  return mag | ((__float_as_uint(x) >> 28) & 8u);
}

// One thread per 16-channel group (bulk: every lane's VALU work is its own).
// Thread gid of a four-lanes-per-group quantisation of `rows` rows of
// `groups` 16-channel groups (the lanes of a group are four consecutive
// lanes of one wave; threads past the job return).  Used by the small-launch
// kernel here and by the extra workgroups of the Full selection launch.
// dst(r): the cache row that source row r is written to (-1: none); the four
// lanes of a group share r, so they take the same branch.
// Four consecutive input values as fp32: fp32 rows, or bf16 rows (the bf16
// bits shifted into the upper half of an fp32 word: exact).
CSA2_DEV void load4(const float* p, float (&v)[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
CSA2_DEV void load4(const uint16_t* p, float (&v)[4]) {
  const u2 w = *reinterpret_cast<const u2*>(p);
  v[0] = __uint_as_float(w[0] << 16); v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16); v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}

template <class T, class Dst>
CSA2_DEV void quantize_quad_thread_to(const T* __restrict__ x, int64_t xs, int64_t rows, int groups,
                                      uint8_t* __restrict__ codes, int64_t cs, uint8_t* __restrict__ scales,
                                      int64_t ss, int64_t gid, Dst dst) {
  if (gid >= rows * groups * 4) return;            // whole quads: the count is a multiple of 4
  const int64_t grp = gid >> 2;
  const int qtr = (int)(gid & 3);
  const int64_t r = grp / groups;
  const int g = (int)(grp - r * groups);
  const int64_t dr = dst(r);
  if (dr < 0) return;
  float v[4];
  load4(x + r * xs + 16 * g + 4 * qtr, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1, 0xF, 0xF, false)));  // xor 1
  amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E, 0xF, 0xF, false)));  // xor 2
  const uint32_t sc = scale_code(amax);
  const float s = e4m3_pos(sc);
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = (s == 0.0f) ? ((__float_as_uint(v[i]) >> 28) & 8u) : element_code(v[i], s);
    bits |= c << (4 * i);
  }
  *reinterpret_cast<uint16_t*>(codes + dr * cs + 8 * g + 2 * qtr) = (uint16_t)bits;
  if (qtr == 0) scales[dr * ss + g] = (uint8_t)sc;
}

template <class T>
CSA2_DEV void quantize_quad_thread(const T* __restrict__ x, int64_t xs, int64_t rows, int groups,
                                   uint8_t* __restrict__ codes, int64_t cs, uint8_t* __restrict__ scales,
                                   int64_t ss, int64_t gid) {
  quantize_quad_thread_to(x, xs, rows, groups, codes, cs, scales, ss, gid, [](int64_t r) { return r; });
}

// Cache row of new row r in a paged cache: position pos[r] of sequence
// seq[r] is row block_table[seq][pos / P] * P + pos % P; -1 when the
// sequence, the position or the page is out of range.
CSA2_DEV int64_t paged_row(const PagedRows& d, int64_t r) {
  const int32_t sq = d.seq[r], t = d.pos[r];
  if (sq < 0 || sq >= d.batch || t < 0 || (t >> d.shift) >= d.max_pages) return -1;
  const int32_t page = d.bt[(int64_t)sq * d.max_pages + (t >> d.shift)];
  const int64_t row = ((int64_t)page << d.shift) + (t & ((1 << d.shift) - 1));
  return page >= 0 && row < d.cache_rows ? row : -1;
}

// one thread of the four-lane quantiser for a job (contiguous or paged rows)
CSA2_DEV void quantize_job_thread(const QuantJob& q, int64_t gid) {
  if (q.pg.bt)
    quantize_quad_thread_to(q.x, q.xs, q.rows, q.groups, q.codes, q.cs, q.scales, q.ss, gid,
                            [&](int64_t r) { return paged_row(q.pg, r); });
  else
    quantize_quad_thread(q.x, q.xs, q.rows, q.groups, q.codes, q.cs, q.scales, q.ss, gid);
}

}  // namespace csa2
