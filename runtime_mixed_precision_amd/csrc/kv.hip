// AutoFP KV cache for gfx950: encoding tokens into base / refinement pages and
// decode attention over them.
//
// "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
// Exponent-Mantissa Refinement" (arXiv 2611.10165v1):
//   §4.1 (last paragraph)  attention reads K/V in the AutoFP construction; two
//                          page types of equal size: T base tokens, or T/2
//                          refined tokens with offsets stored as 4*delta in E2M1
//   §5.1                   KV page size T = 64
//   App. B.1, Eqs. 2-3     NVFP4 encode (T, E4M3 group scales, E2M1 codes)
//   §3.1                   the 2-bit level is for weights only (W2A4KV4)
//
// Attention (one wavefront per (context split, KV head, sequence)):
//   QK   S^T[token][head] = K_hat (16 tokens x 32 dims) . Q^T on
//        v_mfma_f32_16x16x32_f16, K_hat = B*q (+ B*d/8) exact in fp16, the
//        query heads of the KV head in the 16 columns, the query as a sum of
//        two fp16 parts;
//   PV   O^T[dim][head] += V_hat^T (16 dims x 32 tokens) . P^T, same MFMA,
//        V_hat exact in fp16 and P as a sum of two fp16 parts;
//   an online softmax per head between the two (base-2 exponentials), and the
//   tensor scales T_K (in the score scale) and T_V (at the merge) in fp32.
// The token order inside a QK tile is chosen so that the score each lane
// holds is the probability its lane supplies to the PV tile: no data moves
// between the two products. A split's (m, l, O) go to the workspace; a merge
// kernel combines the splits of each (sequence, query head).
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kPageTok = AUTOFP_KV_PAGE_TOKENS;   // base-page capacity
constexpr int kHd = AUTOFP_KV_HEAD_DIM;
constexpr int kSec = AUTOFP_KV_PAGE_BYTES;        // bytes of one KV head of one page
constexpr int kRec = kHd + 4;                     // floats per split record: O, m, l, pad
constexpr int kMaxPagesPerSplit = 64;
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Page write: one thread per (8 consecutive tokens of the call, KV head,
// 16-element group), K and V.
// ---------------------------------------------------------------------------

struct Enc16 {
  uint32_t B;          // E4M3 code
  uint32_t q[16];      // E2M1 codes
  uint32_t o[16];      // E2M1 codes of d/2 (refined tokens)
};

// [AE] App. B.1 Eqs. 2-3 for one group, plus the offsets of [AE] §3.2 stored as
// E2M1 of d/2 ([AE] §4.1): d = +1 -> 0001, 0 -> 0000, -1 -> 1001, -2 -> 1010.
__device__ __forceinline__ void encode_group16(const float *x, float T, float sixT, bool refine,
                                               Enc16 &e) {
#pragma clang fp contract(off)
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  const float b = sixT > 0.0f ? a / sixT : 0.0f;
  e.B = e4m3_encode(b);
  const float s = T * e4m3_value(e.B);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = (s != 0.0f) ? x[i] / s : 0.0f;
    e.q[i] = e2m1_encode(v);
    const uint32_t dc = refine ? offset_code(v - e2m1_value(e.q[i])) : 0u;
    e.o[i] = (0x9A10u >> (4 * dc)) & 0xFu;   // code 0, 1, 2, 3 (d = 0, 1, -2, -1)
  }
}

__device__ __forceinline__ void load16(const void *x, int dtype, int64_t e, float *v) {
  if (dtype == AUTOFP_BF16) {
    const uint4 *p = (const uint4 *)((const uint16_t *)x + e);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint4 w = p[c];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * c + 2 * j] = __uint_as_float(ww[j] << 16);
        v[8 * c + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4 *p = (const float4 *)((const float *)x + e);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 w = p[c];
      v[4 * c] = w.x;
      v[4 * c + 1] = w.y;
      v[4 * c + 2] = w.z;
      v[4 * c + 3] = w.w;
    }
  }
}

__device__ __forceinline__ uint32_t pack8(const uint32_t *c) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= c[i] << (4 * i);
  return w;
}

// Largest value of the partial maxima, by the whole block (identical in every block).
__device__ float block_fold_max(const float *partial, int n) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

constexpr int kWriteThreads = 256;

__global__ __launch_bounds__(kWriteThreads) void kv_write_kernel(KvWriteArgs a) {
#pragma clang fp contract(off)
  float Tk, Tv;
  if (a.set_scale) {
    Tk = block_fold_max(a.k_part, a.n_part) / 2688.0f;
    Tv = block_fold_max(a.v_part, a.n_part) / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *a.k_scale = Tk;
      *a.v_scale = Tv;
    }
  } else {
    Tk = *a.k_scale;
    Tv = *a.v_scale;
  }
  // thread: 8 consecutive tokens of the call, one KV head, one 16-dim group
  const int64_t idx = (int64_t)blockIdx.x * kWriteThreads + threadIdx.x;
  const int64_t nblk = (a.n_tokens + 7) / 8;
  if (idx >= nblk * a.h_kv * (kHd / 16)) return;
  const int j = (int)(idx & 7);
  const int64_t th = idx >> 3;
  const int h = (int)(th % a.h_kv);
  const int64_t t0 = 8 * (th / a.h_kv);
  const int nt = (a.n_tokens - t0) < 8 ? (int)(a.n_tokens - t0) : 8;

  // V fast path: the 8 tokens fill positions 8i .. 8i+7 of one page in order
  // (a prompt), so this thread owns whole V dwords and stores them; otherwise
  // each token merges its nibbles into dwords shared with other tokens
  const int32_t s0 = a.slots[t0];
  bool whole = nt == 8 && s0 >= 0 && (s0 & 7) == 0 && s0 / kPageTok < a.n_pages;
  for (int i = 1; i < 8 && whole; ++i) whole = a.slots[t0 + i] == s0 + i;
  if (whole) whole = (s0 % kPageTok) + 8 <= (a.page_kind[s0 / kPageTok] != 0 ? kPageTok / 2 : kPageTok);
  uint32_t vq[16], vo[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) vq[d] = vo[d] = 0u;

  float x[16];
  Enc16 e;
  for (int i = 0; i < nt; ++i) {
    const int64_t t = t0 + i;
    const int32_t slot = a.slots[t];
    if (slot < 0) continue;
    const int32_t page = slot / kPageTok, pos = slot % kPageTok;
    if (page >= a.n_pages) continue;
    const bool refine = a.page_kind[page] != 0;
    const int cap = refine ? kPageTok / 2 : kPageTok;
    if (pos >= cap) continue;
    const int64_t sec = ((int64_t)page * a.h_kv + h) * kSec;
    const int64_t e0 = (t * a.h_kv + h) * kHd + 16 * j;

    // K: token-major codes, [token][group] scales
    load16(a.k, a.dtype, e0, x);
    encode_group16(x, Tk, 6.0f * Tk, refine, e);
    uint8_t *kp = a.k_pages + sec;
    *(uint2 *)(kp + pos * 64 + 8 * j) = make_uint2(pack8(e.q), pack8(e.q + 8));
    kp[64 * cap + 8 * pos + j] = (uint8_t)e.B;
    if (refine) *(uint2 *)(kp + 72 * cap + pos * 64 + 8 * j) = make_uint2(pack8(e.o), pack8(e.o + 8));

    // V: [token/8][dim/8][dim%8] dwords, each the 8 tokens 8 (token/8) .. + 7
    // of one dim (token t in nibble t % 8), so that a dword is a row of the
    // V_hat^T operand; [group][token] scales
    load16(a.v, a.dtype, e0, x);
    encode_group16(x, Tv, 6.0f * Tv, refine, e);
    uint8_t *vp = a.v_pages + sec;
    const uint32_t sh = 4u * (uint32_t)(pos & 7);
    vp[64 * cap + cap * j + pos] = (uint8_t)e.B;
    if (whole) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        vq[d] |= e.q[d] << sh;
        vo[d] |= e.o[d] << sh;
      }
      continue;
    }
    // dims 16j + d, d = 0..15: blocks 2j and 2j + 1, dword d % 8 of each, i.e.
    // dword d from here; clear the token's nibble, then set it (atomic: other
    // writers of the launch hold the other nibbles)
    uint32_t *vd = (uint32_t *)(vp + ((pos >> 3) * 16 + 2 * j) * 32);
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      atomicAnd(vd + d, ~(0xFu << sh));
      atomicOr(vd + d, e.q[d] << sh);
    }
    if (refine) {
      uint32_t *vr = (uint32_t *)(vp + 72 * cap + ((pos >> 3) * 16 + 2 * j) * 32);
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        atomicAnd(vr + d, ~(0xFu << sh));
        atomicOr(vr + d, e.o[d] << sh);
      }
    }
  }
  if (whole) {
    const int32_t page = s0 / kPageTok, pos = s0 % kPageTok;
    const bool refine = a.page_kind[page] != 0;
    const int cap = refine ? kPageTok / 2 : kPageTok;
    uint8_t *vp = a.v_pages + ((int64_t)page * a.h_kv + h) * kSec;
    uint4 *vd = (uint4 *)(vp + ((pos >> 3) * 16 + 2 * j) * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) vd[q] = make_uint4(vq[4 * q], vq[4 * q + 1], vq[4 * q + 2], vq[4 * q + 3]);
    if (refine) {
      uint4 *vr = (uint4 *)(vp + 72 * cap + ((pos >> 3) * 16 + 2 * j) * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) vr[q] = make_uint4(vo[4 * q], vo[4 * q + 1], vo[4 * q + 2], vo[4 * q + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention over one context split
// ---------------------------------------------------------------------------

// One page's loads for the lane (r = lane % 16, g = lane / 16). Slot 0 holds
// tokens 0..31; slot 1 tokens 32..63 of a base page or the offsets of a
// refinement page (level 6 only). Every page issues the same 14 loads: where
// a refinement page has no slot 1 (level 4), or its slot 1 needs no scales of
// its own, those loads repeat addresses of slot 0 (cache hits), so the number
// of loads in flight is the same on every path and the waits stay exact.
struct PageRegs {
  uint4 kc[2][2];     // [slot][b]: K codes of token tok(b, r), dims 32g .. 32g+31
  uint32_t ks[2][2];  // [slot][b]: the dword of token tok(b, r)'s K scales holding groups 2g, 2g+1
  uint4 vc[2][2];     // [slot][half]: V codes of tokens 8g .. 8g+7, dims 8r .. 8r+7
  uint2 vs[2];        // [slot]: V scales of group r/2, tokens 8g .. 8g+7
};

// Token of row r of QK tile b (of a 32-token slot): 8 (r / 4) + 4 b + r % 4, so
// that the output rows 4g .. 4g+3 of tiles 0 and 1 are tokens 8g .. 8g+7.
__device__ __forceinline__ int qk_token(int b, int r) { return 8 * (r >> 2) + 4 * b + (r & 3); }

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Two E2M1 codes of byte m of w as fp16 (the byte selector must be a constant).
__device__ __forceinline__ half2v fp4_byte(uint32_t w, int m) {
  switch (m) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// Per-lane byte offsets inside a page section, the same for every page.
struct LaneOffsets {
  uint32_t kc[2];     // K codes of token tok(b, r), dims 32g ..
  uint32_t ks[2];     // K scale dword of token tok(b, r) holding groups 2g, 2g+1 (after 64 C)
  uint32_t vc;        // V codes, block (t/8 = g, dim/8 = r)
  uint32_t vs64, vs32;  // V scales of group r/2, tokens 8g.. (after 64 C), for C = 64 and 32
};

__device__ __forceinline__ LaneOffsets lane_offsets(int r, int g) {
  LaneOffsets o;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = qk_token(b, r);
    o.kc[b] = (uint32_t)(t * 64 + 16 * g);
    o.ks[b] = (uint32_t)(8 * t + 4 * (g >> 1));
  }
  o.vc = (uint32_t)((g * 16 + r) * 32);
  o.vs64 = (uint32_t)((r >> 1) * 64 + 8 * g);
  o.vs32 = (uint32_t)((r >> 1) * 32 + 8 * g);
  return o;
}

constexpr int kStream = 2;   // cache policy of the page copies: streamed, non-temporal

// Per wavefront, an LDS ring of two pages: K section at 0, V section at
// kRingV; each section copy is 5 x 1 KB (the last KB ends past the 4608
// section bytes, which read as zeros).
constexpr int kRingV = 5120;
constexpr int kRingPage = 2 * kRingV;
constexpr int kCopyLoads = 10;   // buffer->LDS loads per page

#define KV_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt immediates (gfx9 encoding): vmcnt(10), other counters free; and
// lgkmcnt(0), other counters free.
constexpr int kWaitVm10 = kCopyLoads | (0x7 << 4) | (0xF << 8);
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Copy one page's K and V sections of this KV head into ring slot `dst`
// (memory to LDS, no registers). The bytes a level does not read are left out
// by the resource size: a refinement page's offsets at level 4, and the unused
// tail of a refinement section. The page base is wavefront-uniform (scalar
// registers); lane l copies bytes 16 l + 1024 j. A page that is not live
// (past the split's end, or dropped) issues the same copies over an empty
// range: they write zeros and read no memory.
__device__ __forceinline__ void copy_page(uint8_t *dst, const uint8_t *ks, const uint8_t *vs, bool live,
                                          bool refinement, bool six, int lane) {
  const int bytes = !live ? 0 : refinement ? (six ? 136 * kPageTok / 2 : 72 * kPageTok / 2) : kSec;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(ks), (short)0, bytes,
                                                                      0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(vs), (short)0, bytes,
                                                                      0x00020000);
#pragma unroll
  for (int j = 0; j < 5; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, KV_LDS(dst + 1024 * j), 16, 16 * lane + 1024 * j, 0, 0, kStream);
#pragma unroll
  for (int j = 0; j < 5; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, KV_LDS(dst + kRingV + 1024 * j), 16, 16 * lane + 1024 * j, 0, 0,
                                             kStream);
}

// The lane's operands of one page from its ring slot (the section layout).
// Slot 1 of a refinement page holds its offsets (level 6) or repeats slot 0.
__device__ __forceinline__ void read_page(PageRegs &pr, const uint8_t *src, bool refinement, bool six,
                                          const LaneOffsets &o) {
  const int C = refinement ? kPageTok / 2 : kPageTok;
  const int code1 = refinement ? (six ? 72 * C : 0) : 32 * 64;
  const int ksc1 = refinement ? 0 : 8 * 32;
  const int vsc1 = refinement ? 0 : 32;
  const uint32_t ovs = refinement ? o.vs32 : o.vs64;
  const uint8_t *k = src, *v = src + kRingV;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    pr.kc[0][b] = *(const uint4 *)(k + o.kc[b]);
    pr.kc[1][b] = *(const uint4 *)(k + code1 + o.kc[b]);
    pr.ks[0][b] = *(const uint32_t *)(k + 64 * C + o.ks[b]);
    pr.ks[1][b] = *(const uint32_t *)(k + 64 * C + ksc1 + o.ks[b]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pr.vc[0][h] = *(const uint4 *)(v + o.vc + 16 * h);
    pr.vc[1][h] = *(const uint4 *)(v + code1 + o.vc + 16 * h);
  }
  pr.vs[0] = *(const uint2 *)(v + 64 * C + ovs);
  pr.vs[1] = *(const uint2 *)(v + 64 * C + vsc1 + ovs);
}

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t u4(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct SoftState {
  float m, l;         // reference maximum (base-2 score units) and sum of p of head r
  float4v O[8];       // O[n][i]: head r, dim 32g + 8i + n
};

// Largest step of a stale reference maximum: p = 2^(s - m) stays below 2^8,
// so the fp16 parts of p and the fp32 sums keep their precision.
constexpr float kRescaleSlack = 8.0f;

// Scores of one 32-token slot: x[j] = token 8g + j for head r (base-2 units,
// -inf past `valid`). REF: the slot's offsets are in slot 1 (level 6).
template <bool REF>
__device__ __forceinline__ void qk_slot(const PageRegs &pr, int slot, int valid, const half8v *qb,
                                        const half8v *ql, bool qlo, float cs, int g, float *x) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t sb = (pr.ks[slot][b] >> (16 * (g & 1))) & 0xFFFFu;
    const half2v sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8v k8 = fp4x8_to_half8(u4(pr.kc[slot][b], s));
      if (REF) k8 += fp4x8_to_half8(u4(pr.kc[1][b], s)) * (_Float16)0.25f;
      const _Float16 bs = (s < 2) ? sc[0] : sc[1];
      k8 *= bs;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k8, qb[s], acc, 0, 0, 0);
      if (qlo) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k8, ql[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * b + i;
      x[j] = (8 * g + j < valid) ? acc[i] * cs : -INFINITY;
    }
  }
}

// Online softmax over N scores of head r (N / 8 slots), with the hardware
// base-2 exponential (results below 2^-126, which add nothing next to the
// reference maximum's 1, flush to zero): moves the reference
// maximum only when a score passes it by more than the slack (always on the
// first page, where it is -inf; the result does not depend on it), then
// p = 2^(x - m) as P + Pl, both fp16 (error ~2^-22 p), so the fp16 operand
// rounding of the probabilities does not reach the output.
template <int N>
__device__ __forceinline__ void softmax_update(const float *x, SoftState &st, half8v *P, half8v *Pl) {
  float mb = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) mb = fmaxf(mb, x[j]);
  mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
  mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
  if (__any(mb > st.m + kRescaleSlack)) {
    const float mn = fmaxf(st.m, mb);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
    st.l *= alpha;
    st.m = mn;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.O[n] *= alpha;
  }
  float ps = 0.0f;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - st.m);
    ps += p;
    const _Float16 h = (_Float16)p;
    P[j / 8][j % 8] = h;
    Pl[j / 8][j % 8] = (_Float16)(p - (float)h);
  }
  st.l += ps;
}

// O^T[dim][head] += V_hat^T (16 dims x 32 tokens) . P^T for one slot: output
// tile n holds dims 8r + n; lane (r, g) supplies tokens 8g .. 8g+7 of dim
// 8r + n, one code dword of the page, times the tokens' scales.
template <bool REF>
__device__ __forceinline__ void pv_slot(const PageRegs &pr, int slot, int valid, const half8v &P,
                                        const half8v &Pl, int g, SoftState &st) {
  uint2 vsc = pr.vs[slot];
  const int nv = valid - 8 * g;   // tokens of this lane group that hold data
  if (nv < 8) {
    const uint64_t keep = nv <= 0 ? 0ull : (~0ull >> (64 - 8 * nv));
    vsc.x &= (uint32_t)keep;
    vsc.y &= (uint32_t)(keep >> 32);
  }
  half2v bp[4];   // scales of tokens 2m, 2m + 1 of the lane group
  bp[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc.x, 1.0f, false);
  bp[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc.x, 1.0f, true);
  bp[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc.y, 1.0f, false);
  bp[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc.y, 1.0f, true);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    // dword n of the lane's block: dim 8r + n, tokens 8g .. 8g+7 (byte m =
    // tokens 2m, 2m + 1), already the operand's order
    const uint32_t dv = u4(pr.vc[slot][n >> 2], n & 3);
    half2v c[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      half2v v = fp4_byte(dv, m);
      if (REF) {
        const half2v q4 = half2v{(_Float16)0.25f, (_Float16)0.25f};
        v += fp4_byte(u4(pr.vc[1][n >> 2], n & 3), m) * q4;
      }
      c[m] = v * bp[m];
    }
    const half8v a8 = half8v{c[0][0], c[0][1], c[1][0], c[1][1], c[2][0], c[2][1], c[3][0], c[3][1]};
    st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, P, st.O[n], 0, 0, 0);
    st.O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, Pl, st.O[n], 0, 0, 0);
  }
}

// A base page: its two 32-token slots share one softmax step.
__device__ __forceinline__ void attend_base_page(const PageRegs &pr, int valid, const half8v *qb,
                                                 const half8v *ql, bool qlo, float cs, int g,
                                                 SoftState &st) {
  float x[16];
  qk_slot<false>(pr, 0, valid, qb, ql, qlo, cs, g, x);
  qk_slot<false>(pr, 1, valid - 32, qb, ql, qlo, cs, g, x + 8);
  half8v P[2], Pl[2];
  softmax_update<16>(x, st, P, Pl);
  pv_slot<false>(pr, 0, valid, P[0], Pl[0], g, st);
  pv_slot<false>(pr, 1, valid - 32, P[1], Pl[1], g, st);
}

// A refinement page: one slot of 32 tokens, its offsets in slot 1.
template <bool REF>
__device__ __forceinline__ void attend_refined_page(const PageRegs &pr, int valid, const half8v *qb,
                                                    const half8v *ql, bool qlo, float cs, int g,
                                                    SoftState &st) {
  float x[8];
  qk_slot<REF>(pr, 0, valid, qb, ql, qlo, cs, g, x);
  half8v P[1], Pl[1];
  softmax_update<8>(x, st, P, Pl);
  pv_slot<REF>(pr, 0, valid, P[0], Pl[0], g, st);
}

__global__ __launch_bounds__(64) void kv_attn_split_kernel(KvAttnArgs a) {
  const int split = blockIdx.x, hk = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const int level = a.bits_dev ? *a.bits_dev : a.bits;
  const bool six = level == 6;

  int np = a.seq_pages[b];
  np = np < 0 ? 0 : (np > a.max_pages ? a.max_pages : np);
  const int pps = (np + a.n_split - 1) / a.n_split;
  const int p0 = split * pps;
  const int p1 = (p0 + pps) < np ? (p0 + pps) : np;
  const int npp = p1 > p0 ? p1 - p0 : 0;

  // page id, type and fill of the split's pages, one page per lane; pages
  // without tokens are dropped here (id -1)
  int my_pg = -1, my_kind = 0, my_fill = 0;
  if (lane < npp) {
    const int pg = a.page_table[b * a.max_pages + p0 + lane];
    if (pg >= 0 && pg < a.n_pages) {
      my_kind = a.page_kind[pg] != 0 ? 1 : 0;
      const int cap = my_kind ? kPageTok / 2 : kPageTok;
      const int f = a.page_tokens[pg];
      my_fill = f < 0 ? 0 : (f > cap ? cap : f);
      my_pg = my_fill > 0 ? pg : -1;
    }
  }

  // query fragment: head hk*grp + r (zeros for the unused columns), dims
  // 32g + 8s + 0..7, as fp16 q = qb + ql (ql is zero for bf16 queries in the
  // fp16 range; its MFMA is skipped when the whole wavefront's ql is zero)
  half8v qb[4], ql[4];
  bool any_lo = false;
  {
    const int head = hk * a.grp + r;
    const bool live = r < a.grp;
    const int64_t q0 = (b * a.h_q + (live ? head : 0)) * kHd + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float f[8];
      if (a.q_dtype == AUTOFP_BF16) {
        const uint4 w = *(const uint4 *)((const uint16_t *)a.q + q0 + 8 * s);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = __uint_as_float(ww[j] << 16);
          f[2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
        }
      } else {
        const float4 u = *(const float4 *)((const float *)a.q + q0 + 8 * s);
        const float4 v = *(const float4 *)((const float *)a.q + q0 + 8 * s + 4);
        f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
        f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float fj = live ? f[j] : 0.0f;
        qb[s][j] = (_Float16)fj;
        ql[s][j] = (_Float16)(fj - (float)qb[s][j]);
        any_lo |= ql[s][j] != (_Float16)0.0f;
      }
    }
  }
  const bool qlo = __any(any_lo);
  const float cs = a.sm_scale * *a.k_scale * kLog2e;

  SoftState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.O[n] = float4v{0.f, 0.f, 0.f, 0.f};

  const int64_t head_off = (int64_t)hk * kSec;
  const int64_t page_stride = (int64_t)a.h_kv * kSec;
  // Pages stream through the wavefront's two-page LDS ring: while page i is
  // processed from registers, pages i + 1 and i + 2 are in flight. Page i is
  // read from the ring once its 10 copies have landed (vmcnt(10): only page
  // i + 1's remain), and page i + 2 is copied into the same slot after those
  // reads have returned (lgkmcnt(0)). Past the last page, and for a dropped
  // page (id -1), the copies read nothing (and the page is skipped); every
  // copy has landed before the wavefront ends.
  __shared__ __attribute__((aligned(16))) uint8_t kv_ring0[kRingPage];
  __shared__ __attribute__((aligned(16))) uint8_t kv_ring1[kRingPage];
  const LaneOffsets lo = lane_offsets(r, g);
  auto issue = [&](uint8_t *slot, int i) {
    const bool inside = i < npp;
    i = inside ? i : npp - 1;
    int pg = __builtin_amdgcn_readlane(my_pg, i);
    const int kind = __builtin_amdgcn_readlane(my_kind, i);
    const bool live = inside && pg >= 0;
    pg = pg < 0 ? 0 : pg;
    const uint8_t *kp = a.k_pages + pg * page_stride + head_off;
    const uint8_t *vp = a.v_pages + pg * page_stride + head_off;
    copy_page(slot, kp, vp, live, kind != 0, six, lane);
  };
  auto step = [&](uint8_t *slot, int i) {
    const int pg = __builtin_amdgcn_readlane(my_pg, i);
    const int kind = __builtin_amdgcn_readlane(my_kind, i);
    PageRegs cur;
    __builtin_amdgcn_s_waitcnt(kWaitVm10);
    __builtin_amdgcn_sched_barrier(0);
    read_page(cur, slot, kind != 0, six, lo);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_sched_barrier(0);
    issue(slot, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (pg >= 0) {
      const int valid = __builtin_amdgcn_readlane(my_fill, i);
      if (!kind) attend_base_page(cur, valid, qb, ql, qlo, cs, g, st);
      else if (six) attend_refined_page<true>(cur, valid, qb, ql, qlo, cs, g, st);
      else attend_refined_page<false>(cur, valid, qb, ql, qlo, cs, g, st);
    }
  };
  if (npp > 0) {
    issue(kv_ring0, 0);
    issue(kv_ring1, 1);
    int i = 0;
    for (; i + 1 < npp; i += 2) {
      step(kv_ring0, i);
      step(kv_ring1, i + 1);
    }
    if (i < npp) step(kv_ring0, i);
    __builtin_amdgcn_s_waitcnt(0);
  }

  // split record: O (dims 32g .. 32g+31 of head r), m, l
  float l = st.l + __shfl_xor(st.l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (r < a.grp) {
    float *rec = a.part + ((b * a.h_q + hk * a.grp + r) * a.n_split + split) * kRec;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(float4 *)(rec + 32 * g + 8 * i) = make_float4(st.O[0][i], st.O[1][i], st.O[2][i], st.O[3][i]);
      *(float4 *)(rec + 32 * g + 8 * i + 4) = make_float4(st.O[4][i], st.O[5][i], st.O[6][i], st.O[7][i]);
    }
    if (g == 0) {
      rec[kHd] = st.m;
      rec[kHd + 1] = l;
    }
  }
}

// Combine the splits of one (sequence, query head): one wavefront, two dims per
// lane. Lane s holds split s's (m, l) and its weight 2^(m_s - M); the output
// loop then issues the splits' O loads eight at a time (n_split <= 64).
__global__ __launch_bounds__(64) void kv_attn_merge_kernel(const float *__restrict__ part, int n_split,
                                                           const float *__restrict__ v_scale,
                                                           float *__restrict__ out) {
  const int64_t row = blockIdx.x;
  const float *rec0 = part + row * n_split * kRec;
  const int lane = threadIdx.x;
  const float ms = lane < n_split ? rec0[lane * kRec + kHd] : -INFINITY;
  const float ls = lane < n_split ? rec0[lane * kRec + kHd + 1] : 0.0f;
  const float M = wave_max(ms);
  const float w = (M != -INFINITY && ms != -INFINITY) ? exp2f(ms - M) : 0.0f;
  float L = ls * w;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) L += __shfl_xor(L, d, 64);
  float o0 = 0.0f, o1 = 0.0f;
  for (int s0 = 0; s0 < n_split; s0 += 8) {
    float2 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = s0 + j < n_split ? s0 + j : n_split - 1;
      o[j] = *(const float2 *)(rec0 + sj * kRec + 2 * lane);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = __shfl(w, s0 + j, 64);   // 0 past n_split (lanes >= n_split hold w = 0)
      o0 += o[j].x * wj;
      o1 += o[j].y * wj;
    }
  }
  const float f = L > 0.0f ? *v_scale / L : 0.0f;
  *(float2 *)(out + row * kHd + 2 * lane) = make_float2(o0 * f, o1 * f);
}

}  // namespace

// Context splits per (sequence, KV head): about 8192 / rows, i.e. one round
// of two wavefronts per SIMD (2048 wavefronts) at four query heads per KV
// head. 16 x 32768 tokens, 32/8 heads: 16 splits of 32 pages, 139 us at
// level 4, against 153 us with 32 splits (two rounds) and 162 us with 64.
int kv_attn_splits(int64_t rows, int64_t max_pages) {
  int64_t s = (8192 + rows - 1) / rows;
  const int64_t need = (max_pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit;
  if (s < need) s = need;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > max_pages) s = max_pages;
  if (s < 1) s = 1;
  return (int)s;
}

int64_t kv_attn_max_pages() { return (int64_t)kMaxSplits * kMaxPagesPerSplit; }

size_t kv_attn_workspace_bytes(int64_t rows, int64_t max_pages) {
  return (size_t)rows * (size_t)kv_attn_splits(rows, max_pages) * kRec * sizeof(float);
}

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s) {
  const int64_t n = (a.n_tokens + 7) / 8 * a.h_kv * (kHd / 16);
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)((n + kWriteThreads - 1) / kWriteThreads)),
                     dim3(kWriteThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_attention(const KvAttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(kv_attn_split_kernel, dim3((unsigned)a.n_split, (unsigned)a.h_kv, (unsigned)a.batch),
                     dim3(64), 0, s, a);
  hipLaunchKernelGGL(kv_attn_merge_kernel, dim3((unsigned)(a.batch * a.h_q)), dim3(64), 0, s, a.part,
                     a.n_split, a.v_scale, a.out);
  return hipGetLastError();
}

}  // namespace afp
