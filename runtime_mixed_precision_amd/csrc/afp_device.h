// Device-side helpers of the AutoFP kernels for gfx950: element/scale codecs,
// packed-operand conversions and wave reductions.
//
// Formats ("AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via
// Automatic Exponent-Mantissa Refinement", arXiv 2611.10165v1, App. B,
// Tables 5-6):
//   E2M1 element  s|e1|e0|m, bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3 scale    OCP E4M3FN, bias 7, subnormals m * 2^-9, max 448
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afp {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Scalar codecs (encode side; exact IEEE fp32, no contraction)
// ---------------------------------------------------------------------------

// E4M3 value of a scale code; the sign bit is ignored (scales are magnitudes).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  code &= 0x7F;
  const uint32_t e = code >> 3, m = code & 7;
  if (e == 0) return (float)m * 0.001953125f;        // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Nearest E4M3 code to b >= 0 (round half to even), saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float b) {
  if (!(b < 448.0f)) return 0x7Eu;
  if (b < 0.015625f) {                                 // below 2^-6: step 2^-9
    return (uint32_t)rintf(b * 512.0f);                // 0..8 (8 = code of 2^-6)
  }
  uint32_t u = __float_as_uint(b);
  u += 0x7FFFFu + ((u >> 20) & 1u);                    // round mantissa to 3 bits, ties even
  const uint32_t code = (u >> 20) - (120u << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 magnitude index of |v| with round half to even: the decision points are
// the midpoints 0.25 .. 5; a tie goes to the even index (mantissa bit 0).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  const uint32_t i = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return i ? (i | ((__float_as_uint(v) >> 28) & 8u)) : 0u;   // canonical +0
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
  return (c & 8u) ? -mag : mag;
}

// Signed offset for a residual r = v - q: argmin over d in {-2,-1,0,1} of
// |r - d/8|, ties to the smaller |d|. Returned as its 2-bit two's-complement code.
__device__ __forceinline__ uint32_t offset_code(float r) {
  const int d = (r > 0.0625f) ? 1 : (r >= -0.0625f) ? 0 : (r >= -0.1875f) ? -1 : -2;
  return (uint32_t)d & 3u;
}

// Offset variants ("AutoEMatic" App. I: 4-bit offsets, AutoFP8; §6.5 /
// Fig. 14(a): the step 2^(e-3) of the element's own exponent).
//
// 2^-e for the unbiased exponent e = max(field - 1, 0) of an E2M1 code's value
// (fields 00 and 01 give e = 0, 10 gives 1, 11 gives 2): argmin over d of
// |r - d 2^(e-3)| = argmin |r 2^-e - d/8|, the scaling being exact.
__device__ __forceinline__ float e2m1_inv_pow2e(uint32_t code) {
  const uint32_t f = (code >> 1) & 3u;
  return f == 3u ? 0.25f : (f == 2u ? 0.5f : 1.0f);
}

// 4-bit signed offset: argmin over d in -8..7 of |r - d/8|, ties to the
// smaller |d| (u = 8r is exact; |u| - 0.5 is exact for these magnitudes).
__device__ __forceinline__ int offset8(float r) {
  const float u = 8.0f * r;
  const int m = (int)ceilf(fabsf(u) - 0.5f);
  const int d = u < 0.0f ? -m : m;
  return d < -8 ? -8 : (d > 7 ? 7 : d);
}

// E2M3 (FP6g element, bias 1, max 7.5) code of v with round half to even on
// the code (the grid steps 1/8 below 2, 1/4 on [2, 4), 1/2 on [4, 7.5]);
// saturates at 7.5; canonical +0. Every subtraction and scaling is exact.
__device__ __forceinline__ uint32_t e2m3_encode(float v) {
  const float a = fabsf(v);
  uint32_t c;
  if (!(a < 7.5f)) c = 31u;
  else if (a < 2.0f) c = (uint32_t)rintf(a * 8.0f);                     // 0..16 (16 = 2.0)
  else if (a < 4.0f) c = 16u + (uint32_t)rintf((a - 2.0f) * 4.0f);       // 16..24
  else c = 24u + (uint32_t)rintf((a - 4.0f) * 2.0f);                     // 24..31
  return c ? (c | ((__float_as_uint(v) >> 26) & 32u)) : 0u;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Packed-operand conversions (compute side)
// ---------------------------------------------------------------------------

// Eight E2M1 codes of one dword (element 2i in the low nibble of byte i) to
// eight fp16 values, via the gfx950 fp4 converts with unit scale (exact).
__device__ __forceinline__ half8v fp4x8_to_half8(uint32_t w) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return half8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four fp16 offsets d/8 of one offset byte (2-bit codes 00 -> 0, 01 -> +1/8,
// 10 -> -1/4, 11 -> -1/8), as two packed half2 words. Branch-free: the four
// fp16 values have a zero low byte, so a byte permute of the table of their
// high bytes (code 0: 0x00, 1: 0x30, 2: 0xB4, 3: 0xB0) builds two of them per
// word (selector 0x0C gives a zero byte).
__device__ __forceinline__ uint2 delta_words(uint32_t byte) {
  constexpr uint32_t kHi = 0xB0B43000u;
  const uint32_t c0 = byte & 3u, c1 = (byte >> 2) & 3u, c2 = (byte >> 4) & 3u, c3 = (byte >> 6) & 3u;
  const uint32_t s01 = 0x000C000Cu | (c0 << 8) | (c1 << 24);
  const uint32_t s23 = 0x000C000Cu | (c2 << 8) | (c3 << 24);
  return make_uint2(__builtin_amdgcn_perm(kHi, kHi, s01), __builtin_amdgcn_perm(kHi, kHi, s23));
}

// AutoFP2 digit codes from eight E2M1 codes: keep the sign, magnitude bits
// {e1 AND e0, e1 XOR e0} placed as the E2M1 codes of 2 (0b100) and 1 (0b010).
__device__ __forceinline__ uint32_t autofp2_codes(uint32_t w) {
  const uint32_t e1 = (w >> 2) & 0x11111111u;
  const uint32_t e0 = (w >> 1) & 0x11111111u;
  return (w & 0x88888888u) | ((e1 & e0) << 2) | ((e1 ^ e0) << 1);
}

// fp16 offsets of one offset byte: d_e / 8 for elements e = 0..3.
__device__ __forceinline__ void offsets_to_half4(uint32_t byte, half2v &lo, half2v &hi) {
  auto dv = [](uint32_t c) -> _Float16 {
    const int d = (int)(c & 3u) - (int)((c & 2u) << 1);   // sign-extend 2 bits
    return (_Float16)((float)d * 0.125f);
  };
  lo = half2v{dv(byte), dv(byte >> 2)};
  hi = half2v{dv(byte >> 4), dv(byte >> 6)};
}

// Variant formats (compute side). 2^e of the E2M1 values in h (e = the
// unbiased exponent, 0 below 1): the exponent bits of each fp16 value with a
// zero mantissa, at least 1.0; the exponent-scaled offset is d/8 times it.
__device__ __forceinline__ half2v pow2e_h2(half2v q) {
  const uint32_t u = __builtin_bit_cast(uint32_t, q);
  uint32_t lo = u & 0x7C00u, hi = (u >> 16) & 0x7C00u;
  lo = lo > 0x3C00u ? lo : 0x3C00u;
  hi = hi > 0x3C00u ? hi : 0x3C00u;
  return __builtin_bit_cast(half2v, lo | (hi << 16));
}

// d/8 of a 4-bit two's-complement offset (AutoFP8), d clamped to [-2, +1]
// when `clamp6` (the same tensor at level 6); exact in fp16.
__device__ __forceinline__ _Float16 delta8_h(uint32_t nib, bool clamp6) {
  int d = (int)(nib & 15u) - (int)((nib & 8u) << 1);
  if (clamp6) d = d < -2 ? -2 : (d > 1 ? 1 : d);
  return (_Float16)((float)d * 0.125f);
}

// fp16 values of two 6-bit E2M3 codes (FP6g): the code's five magnitude bits
// at fp16 bits [11:7] read 2^(e-15) (1 + m/8) for e > 0 and m 2^-17 for e = 0;
// times 2^14 they are 2^(e-1) (1 + m/8) and m/8, the E2M3 values (exact).
__device__ __forceinline__ half2v e2m3x2_to_half2(uint32_t c0, uint32_t c1) {
  auto bits = [](uint32_t c) -> uint32_t { return ((c & 0x20u) << 10) | ((c & 0x1Fu) << 7); };
  const half2v raw = __builtin_bit_cast(half2v, bits(c0) | (bits(c1) << 16));
  return raw * half2v{(_Float16)16384.0f, (_Float16)16384.0f};
}

// ---------------------------------------------------------------------------
// Wave reductions (64-wide wavefronts)
// ---------------------------------------------------------------------------

// Largest value of the wavefront in every lane (fmaxf: NaNs are skipped),
// through DPP row moves and the gfx950 row swaps (no LDS permutes).
__device__ __forceinline__ float wave_max(float v) {
  auto dmax = [](float x, int ctrl) -> float {
    int y = 0;
    switch (ctrl) {   // the DPP control must be a constant
      case 0: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false); break;   // quad xor 1
      case 1: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false); break;   // quad xor 2
      case 2: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false); break;  // row half mirror
      default: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return fmaxf(x, __int_as_float(y));
  };
  v = dmax(v, 0);
  v = dmax(v, 1);
  v = dmax(v, 2);
  v = dmax(v, 3);   // every lane: max of its row of 16
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));   // rows (0, 1) and (2, 3)
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Largest value of the wavefront in every lane, through DPP row moves and the
// gfx950 row swaps (no LDS traffic, ALU latency only).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto dmax = [](uint32_t x, int ctrl) -> uint32_t {
    uint32_t y = 0;
    switch (ctrl) {   // the DPP control must be a constant
      case 0: y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false); break;   // quad xor 1
      case 1: y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false); break;   // quad xor 2
      case 2: y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false); break;  // row half mirror
      default: y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return x > y ? x : y;
  };
  v = dmax(v, 0);
  v = dmax(v, 1);
  v = dmax(v, 2);
  v = dmax(v, 3);   // every lane: max of its row of 16
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] > a[1] ? a[0] : a[1];   // max of rows (0, 1) and of rows (2, 3)
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] > b[1] ? b[0] : b[1];
}

// Order-preserving map of fp32 to uint32 (for -inf < ... < +inf; NaN unordered).
__device__ __forceinline__ uint32_t f32_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of the wavefront's fp64 values through DPP row moves and the gfx950
// row swaps (ALU latency only: no LDS permutes). Every lane ends with a sum of
// all 64 values; lane 0's is formed in one fixed order (quad pairs, quads,
// half rows, rows, row pairs, halves), so it does not vary between runs.
__device__ __forceinline__ double wave_sum_d_dpp(double v) {
  auto move = [](double x, int ctrl) -> double {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    switch (ctrl) {   // the DPP control must be a constant
      case 0: lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false); break;
      case 1: lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false); break;
      case 2: lo = __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, false); break;
      default: lo = __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, false); hi = __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  };
  v += move(v, 0);   // quad xor 1
  v += move(v, 1);   // quad xor 2: the quad's sum
  v += move(v, 2);   // half-row mirror: 8 lanes
  v += move(v, 3);   // row mirror: 16 lanes
  auto swap_add = [](double x, bool rows32) -> double {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto l = rows32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                          : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = rows32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                          : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    // the pair holds this lane's value and its partner's; fp addition commutes
    return __builtin_bit_cast(double, ((uint64_t)h[0] << 32) | l[0]) +
           __builtin_bit_cast(double, ((uint64_t)h[1] << 32) | l[1]);
  };
  v = swap_add(v, false);   // rows (0, 1) and (2, 3)
  return swap_add(v, true); // halves
}

}  // namespace afp
