// Device-side AutoFP encode of one subgroup and the producer-epilogue
// elementwise ops of the encode kernels.
//
// "AutoEMatic" (arXiv 2611.10165v1): App. B.1 Eqs. 2-3 (NVFP4 base), §3.2
// (AutoFP6 offsets and masks), §6.4 (activation refinement outside M_W;
// the post-processing unit's non-linear operations), App. B.2 (FP6g),
// App. I (AutoFP8), §6.5 / Fig. 14(a) (exponent-scaled offsets).
#pragma once

#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

// ---------------------------------------------------------------------------
// Producer epilogue ([AE] §6.4: the post-processing unit turns completed
// outputs into the next layer's input activations, non-linear operations
// included): four consecutive elements j .. j + 3 of row r of
//   COPY      v = z[r][j]                         (the first k columns of z)
//   RESIDUAL  v = resid[r][j] + z[r][j]
//   SWIGLU    v = silu(z[r][j]) * z[r][k + j],    silu(g) = g / (1 + e^-g)
//   RESIDUAL_RMSNORM  v = (resid[r][j] + z[r][j]) * c[r]   (c: the row's RMSNorm scale)
// in fp32; silu within a few units in the last place (below).
// ---------------------------------------------------------------------------

// silu(g) = g / (1 + e^-g): e^-g = 2^t with t = -g log2(e) carried as
// t_hi + t_lo (log2(e) split into two fp32 parts, the product's rounding
// error recovered by an fma), 2^t_hi from the hardware exp2 (1 ulp) times the
// first-order correction (1 + t_lo ln 2), then the hardware reciprocal
// (1 ulp) and one product: relative error below 4 * 2^-23. Past t_hi = 128
// (g < -88.7) e^-g overflows and the result is -0, as with expf.
__device__ __forceinline__ float silu_f32(float g) {
#pragma clang fp contract(off)
  constexpr float kL2eHi = 1.44269502162933349609375f;   // fp32(log2 e)
  constexpr float kL2eLo = 1.9259629912e-08f;            // log2 e - kL2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float th = -g * kL2eHi;
  const float tl = fmaf(-g, kL2eHi, -th) + (-g) * kL2eLo;
  const float eh = __builtin_amdgcn_exp2f(th);
  const float e = th < 128.0f ? fmaf(eh, tl * kLn2, eh) : eh;
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// u = resid + z of the residual ops (the RESIDUAL_RMSNORM hidden state)
__device__ __forceinline__ float4 resid_sum4(const EncodeArgs &a, int64_t r, int64_t j) {
#pragma clang fp contract(off)
  const float4 zz = *(const float4 *)(a.z + r * a.ldz + j);
  const float4 rr = *(const float4 *)(a.resid + r * a.k + j);
  return make_float4(rr.x + zz.x, rr.y + zz.y, rr.z + zz.z, rr.w + zz.w);
}

__device__ __forceinline__ float4 scale4(float4 u, float c) {
#pragma clang fp contract(off)
  return make_float4(u.x * c, u.y * c, u.z * c, u.w * c);
}

__device__ __forceinline__ float4 epilogue4(const EncodeArgs &a, int64_t r, int64_t j) {
#pragma clang fp contract(off)
  if (a.op == AUTOFP_EPI_RESIDUAL_RMSNORM) return scale4(resid_sum4(a, r, j), a.rowscale[r]);
  const float4 zz = *(const float4 *)(a.z + r * a.ldz + j);
  if (a.op == AUTOFP_EPI_RESIDUAL) {
    const float4 rr = *(const float4 *)(a.resid + r * a.k + j);
    return make_float4(rr.x + zz.x, rr.y + zz.y, rr.z + zz.z, rr.w + zz.w);
  }
  if (a.op == AUTOFP_EPI_SWIGLU) {
    const float4 u = *(const float4 *)(a.z + r * a.ldz + a.k + j);
    return make_float4(silu_f32(zz.x) * u.x, silu_f32(zz.y) * u.y, silu_f32(zz.z) * u.z, silu_f32(zz.w) * u.w);
  }
  return zz;
}

__device__ __forceinline__ float max4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float quad_max(float v) {
  const float a = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v = fmaxf(v, a);
  const float b = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return fmaxf(v, b);
}

// Encode of subgroup s (4 elements x) of row `row` once T is known: E2M1
// codes, the group's E4M3 scale, and the format's offsets and masks. Every
// lane of the wavefront calls it (quad max, ballot); the subgroups of a
// wavefront are 64 consecutive subgroups of one row, lane l holding one with
// s = l (mod 64). ex: the subgroup is in the exclusion mask; wbyte / wpos: the
// weight-mask byte of s and the compacted position of s in its row.
__device__ __forceinline__ void encode_subgroup(const EncodeArgs &a, float T, int64_t row, int64_t s,
                                                bool live, float4 x4, uint32_t ex, uint32_t wbyte,
                                                int32_t wpos) {
#pragma clang fp contract(off)
  const float x[4] = {x4.x, x4.y, x4.z, x4.w};
  const float sixT = 6.0f * T;
  const int64_t ns = a.k / 4;                                  // subgroups per row
  const int64_t mb = (a.k + 31) / 32;                          // mask bytes per row
  const int lane = threadIdx.x & 63;
  const bool want_act = a.act_refine != 0;
  const bool want_w = a.w_mask != nullptr;
  // group scale (the quad's 16 elements)
  const float gm = quad_max(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
  const float b = sixT > 0.0f ? gm / sixT : 0.0f;
  const uint32_t B = e4m3_encode(b);
  const float sc = T * e4m3_value(B);
  float v[4];
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (sc != 0.0f) ? x[i] / sc : 0.0f;
    q[i] = e2m1_encode(v[i]);
  }
  if (live) {
    *(uint16_t *)(a.codes + row * (a.k / 2) + 2 * s) = (uint16_t)(q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12));
    if ((s & 3) == 0) a.scales[row * (a.k / 16) + (s >> 2)] = (uint8_t)B;
  }
  if (!want_act && !want_w) return;

  // offsets d = argmin |r - d step|, r = v - q (exact in fp32): 2-bit codes
  // (step 1/8, or 2^(e-3) for the exponent-scaled format), one byte per
  // subgroup; AutoFP8: 4-bit codes (step 1/8), two bytes per subgroup
  uint32_t ob = 0;
  if (a.fmt == AUTOFP_FMT_AUTOFP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ob |= ((uint32_t)offset8(v[i] - e2m1_value(q[i])) & 15u) << (4 * i);
  } else if (a.fmt == AUTOFP_FMT_AUTOFP6E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ob |= offset_code((v[i] - e2m1_value(q[i])) * e2m1_inv_pow2e(q[i])) << (2 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) ob |= offset_code(v[i] - e2m1_value(q[i])) << (2 * i);
  }
  const bool wide = a.fmt == AUTOFP_FMT_AUTOFP8;

  if (want_act) {
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = v[i] - e2m1_value(q[i]);
      const float rr = r * r;
      const float vv = v[i] * v[i];
      num = (i == 0) ? rr : num + rr;
      den = (i == 0) ? vv : den + vv;
    }
    const float thr = a.thresh * den;
    const bool refine = live && den > 0.0f && num > thr && !ex;
    const uint64_t bits = __ballot(refine);
    if (live) {
      if (wide) *(uint16_t *)(a.act_offsets + row * 2 * ns + 2 * s) = (uint16_t)(refine ? ob : 0u);
      else a.act_offsets[row * ns + s] = (uint8_t)(refine ? ob : 0u);
      if ((s & 7) == 0) a.act_mask[row * mb + (s >> 3)] = (uint8_t)(bits >> lane);
    }
  }
  // the mask's popcount should equal n_refined; a mask with more refined
  // subgroups writes only the first n_refined of each row
  if (want_w && live && ((wbyte >> (s & 7)) & 1u) && wpos < a.n_refined) {
    if (wide) *(uint16_t *)(a.w_offsets + (row * (int64_t)a.n_refined + wpos) * 2) = (uint16_t)ob;
    else a.w_offsets[row * (int64_t)a.n_refined + wpos] = (uint8_t)ob;
  }
}

// FP6g ([AE] App. B.2): Eqs. 2-3 with the E2M3 maximum 7.5 in place of 6,
// T = amax / (7.5 * 448), B_j = E4M3(amax_j / (7.5 T)), q_i = E2M3(x_i / (T B_j));
// four 6-bit codes in three bytes (code i of a subgroup at bits 6i..6i+5 of a
// little-endian 24-bit word). Called like encode_subgroup.
__device__ __forceinline__ void encode_subgroup_fp6g(const EncodeArgs &a, float T, int64_t row, int64_t s,
                                                     bool live, float4 x4) {
#pragma clang fp contract(off)
  const float x[4] = {x4.x, x4.y, x4.z, x4.w};
  const float sevT = 7.5f * T;
  const float gm = quad_max(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
  const float b = sevT > 0.0f ? gm / sevT : 0.0f;
  const uint32_t B = e4m3_encode(b);
  const float sc = T * e4m3_value(B);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) word |= e2m3_encode((sc != 0.0f) ? x[i] / sc : 0.0f) << (6 * i);
  if (live) {
    uint8_t *c = a.codes + row * (3 * a.k / 4) + 3 * s;
    c[0] = (uint8_t)word;
    c[1] = (uint8_t)(word >> 8);
    c[2] = (uint8_t)(word >> 16);
    if ((s & 3) == 0) a.scales[row * (a.k / 16) + (s >> 2)] = (uint8_t)B;
  }
}

// tensor scale T = amax / (max element * 448)
__device__ __forceinline__ float tensor_scale_of(const EncodeArgs &a, float amax) {
  return a.fmt == AUTOFP_FMT_FP6G ? amax / 3360.0f : amax / 2688.0f;
}

// The four elements of subgroup s of row `row` of the tensor to encode (x,
// or the epilogue's v).
__device__ __forceinline__ float4 load_quad(const EncodeArgs &a, int64_t row, int64_t s) {
  if (a.op) return epilogue4(a, row, 4 * s);
  const int64_t e = row * a.k + 4 * s;
  if (a.dtype == AUTOFP_BF16) {
    const uint2 p = *(const uint2 *)((const uint16_t *)a.x + e);
    return make_float4(__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xFFFF0000u),
                       __uint_as_float(p.y << 16), __uint_as_float(p.y & 0xFFFF0000u));
  }
  return *(const float4 *)((const float *)a.x + e);
}

// The same with the source fixed at compile time: 0 x fp32, 1 x bf16, or
// 1 + the epilogue op (2 copy, 3 residual, 4 SwiGLU, 5 residual + RMSNorm
// with the row scales in a.rowscale).
template <int SRC>
__device__ __forceinline__ float4 load_quad_t(const EncodeArgs &a, int64_t row, int64_t s) {
  if constexpr (SRC >= 2) {
    return epilogue4(a, row, 4 * s);
  } else if constexpr (SRC == 1) {
    const uint2 p = *(const uint2 *)((const uint16_t *)a.x + row * a.k + 4 * s);
    return make_float4(__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xFFFF0000u),
                       __uint_as_float(p.y << 16), __uint_as_float(p.y & 0xFFFF0000u));
  } else {
    return *(const float4 *)((const float *)a.x + row * a.k + 4 * s);
  }
}

}  // namespace afp
