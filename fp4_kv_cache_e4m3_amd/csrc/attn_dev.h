// Device helpers shared by the CSA2 attention kernels for gfx950 (not part of
// the ABI): LDS transposes, cross-lane maxima, FP4 / E4M3 decoding, buffer
// resources and the QK^T MFMA step.
#pragma once

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

// Two E4M3 scale bytes of w (chosen by the v_perm selector sel, which puts
// them at bytes 0 and 2) -> fp16 values scale * 2^-8.  A scale byte has sign
// 0; shifted left by 7 it puts its 4 exponent and 3 mantissa bits in fp16's
// fields, where the exponent bias is 15 instead of 7: the fp16 value is the
// scale times 2^-8, subnormal scales included.
CSA2_DEV v2h e4m3_pair_s8(uint32_t w, uint32_t sel) {
  return __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0u, w, sel) << 7);
}

// Eight FP4 codes -> fp16 times an E4M3 scale s, given s8 = s * 2^-8 in fp16:
// the conversion scales the codes by 2^8 (a power of two: exact) and one
// packed multiply applies s8.  code * 2^8 and s * 2^-8 are exact in fp16, and
// so is their product code * s (at most 5 significant bits, inside fp16's
// range), so the result equals the FP4 value times the scale exactly.
CSA2_DEV v8h fp4x8_to_half_s8(uint32_t x, _Float16 s8) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 0);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 1);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 2);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 3);
  const v8h v = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  const v8h sv = {s8, s8, s8, s8, s8, s8, s8, s8};
  return v * sv;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over [base, base + bytes): loads past the end return zeros.
CSA2_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// QK^T k-step in the operands' own type (products exact, fp32 accumulation)
CSA2_DEV v4f mfma_qk(v8h a, v8h b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
CSA2_DEV v4f mfma_qk(v8bf a, v8bf b, v4f c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

}  // namespace csa2
