// Activation decode of the variant formats, shared by the fp16 panel pass
// (gemv.hip) and the variant GEMV's block prologue (gemm.hip).
#pragma once

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

// The variant formats' activation decode of 8 consecutive elements:
// AUTOFP6E B (q + d 2^(e-3)), AUTOFP8 B (q + d/8) (d clamped to [-2, +1] at
// level 6), FP6G B q with E2M3 codes; `refine` adds the offsets.
__device__ __forceinline__ uint4 act_decode8_fmt(const LinearArgs &a, int64_t tok, int64_t k0, bool refine,
                                                 int level) {
  if (k0 >= a.k) return make_uint4(0, 0, 0, 0);
  half2v h[4];
  if (a.fmt == AUTOFP_FMT_FP6G) {
    // 8 codes in 6 bytes (2-byte aligned)
    const uint16_t *c16 = (const uint16_t *)(a.x_codes + tok * (3 * a.k / 4) + (3 * k0 / 4));
    const uint64_t w = (uint64_t)c16[0] | ((uint64_t)c16[1] << 16) | ((uint64_t)c16[2] << 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = e2m3x2_to_half2((uint32_t)(w >> (12 * i)) & 63u, (uint32_t)(w >> (12 * i + 6)) & 63u);
  } else {
    const uint32_t cw = *(const uint32_t *)(a.x_codes + tok * (a.k >> 1) + (k0 >> 1));
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3);
    if (refine && a.fmt == AUTOFP_FMT_AUTOFP6E) {
      const uint32_t ob = *(const uint16_t *)(a.x_offsets + tok * (a.k >> 2) + (k0 >> 2));
      const uint2 d0 = delta_words(ob & 0xFFu), d1 = delta_words(ob >> 8);
      h[0] += __builtin_bit_cast(half2v, d0.x) * pow2e_h2(h[0]);
      h[1] += __builtin_bit_cast(half2v, d0.y) * pow2e_h2(h[1]);
      h[2] += __builtin_bit_cast(half2v, d1.x) * pow2e_h2(h[2]);
      h[3] += __builtin_bit_cast(half2v, d1.y) * pow2e_h2(h[3]);
    } else if (refine && a.fmt == AUTOFP_FMT_AUTOFP8) {
      // two bytes per subgroup: element e of these 8 at bits [4e+3:4e]
      const uint32_t ow = *(const uint32_t *)(a.x_offsets + tok * (a.k >> 1) + (k0 >> 1));
      const bool c6 = level == 6;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] += half2v{delta8_h(ow >> (8 * i), c6), delta8_h(ow >> (8 * i + 4), c6)};
    }
  }
  const _Float16 B = (_Float16)e4m3_value(a.x_scales[tok * (a.k >> 4) + (k0 >> 4)]);
  const half2v b2 = half2v{B, B};
  return make_uint4(__builtin_bit_cast(uint32_t, h[0] * b2), __builtin_bit_cast(uint32_t, h[1] * b2),
                    __builtin_bit_cast(uint32_t, h[2] * b2), __builtin_bit_cast(uint32_t, h[3] * b2));
}

}  // namespace afp
