// Decode-phase AutoFP linear layer (GEMV, up to 64 tokens per launch) for gfx950.
//
// "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
// Exponent-Mantissa Refinement" (arXiv 2611.10165v1), §3.1-3.2 and §4: a layer
// runs at level 2 (AutoFP2 weights c*T*B*Q, NVFP4 activations), 4 (NVFP4 x
// NVFP4) or 6 (both operands refined, T*B*(q + d/8)). The result is the
// product of the decoded operands.
//
// Exactness: a decoded operand without its tensor scale, B*(q + d/8), has at
// most 10 significant bits and lies in [2^-12, 2744], so it is exact in fp16.
// The matrix cores (v_mfma_f32_16x16x32_f16) form exact products and add them
// in fp32; T_W*T_A (and c for level 2) is applied once per output. This
// replaces the pages' extended-K construction: the refinement is folded into
// the operand instead of a second reduction segment.
//
// Work split (streaming kernel): one block owns 16 weight rows and the whole
// K; its W wavefronts split K into contiguous ranges of 256-element chunks.
// In a chunk, lane l handles weight row l%16 and the 64 elements
// [64*(l/16), 64*(l/16)+64): 32 bytes of codes (two 16-byte loads, so the 4
// lanes of a row read one full 128-byte line), 4 scale bytes (one dword) and,
// at level 6, a window of up to 8 compacted offset bytes. Each wavefront keeps
// kInflight chunks of loads in flight. The activation operand comes from an
// fp16 copy of the decoded activations: in LDS when it fits (the block decodes
// it once, overlapped with the first weight loads), otherwise from an fp16
// panel in the workspace that a small pre-pass writes. Partial 16x16 tiles of
// the wavefronts are summed in LDS.
//
// Level-6 weight offsets: the weight mask is shared by every row, so the
// position of a lane's offset bytes in each row's compacted array is the same
// for all rows. Each wavefront derives, once, for every (chunk, lane group)
// of its range: the number of refined subgroups before it and a byte selector
// per subgroup slot. In the loop a lane loads its 8-byte offset window with
// three aligned dword loads, expands it to one byte per slot with v_perm, and
// adds the fp16 offsets d/8 of each refined slot from a 256-entry LDS table.
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kCh = 256;         // K elements per chunk
constexpr int kInflight = 4;     // chunks of weight loads in flight per wavefront
constexpr int kMaxWaves = 16;    // wavefronts per block (1024 threads)
constexpr int kPlanChunks = 16;  // chunks per wavefront covered by one offset plan
static_assert(kPlanChunks % kInflight == 0, "plan rounds must start at a load group");

__device__ __forceinline__ int run_level(const LinearArgs &a) {
  return a.bits_dev ? *a.bits_dev : a.bits;
}

// fp16 bit pattern of d/8 for a 2-bit offset code: 00 -> 0, 01 -> +1/8,
// 10 -> -1/4, 11 -> -1/8.
__device__ __forceinline__ uint32_t delta_bits(uint32_t c) {
  return c == 0 ? 0u : c == 1 ? 0x3000u : c == 2 ? 0xB400u : 0xB000u;
}

// Four fp16 offsets of one offset byte, as two packed half2 words.
__device__ __forceinline__ uint2 delta_words(uint32_t byte) {
  return make_uint2(delta_bits(byte & 3u) | (delta_bits((byte >> 2) & 3u) << 16),
                    delta_bits((byte >> 4) & 3u) | (delta_bits((byte >> 6) & 3u) << 16));
}

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// AutoFP2 remap of eight E2M1 codes ([AE] §3.2): the magnitude index
// i = e1 e0 m maps to the digit Q = (i + 2) >> 2 (0,0,1,1,1,1,2,2), stored as
// the E2M1 code of Q (0b000, 0b010, 0b100); the sign bit is kept.
__device__ __forceinline__ uint32_t autofp2_remap(uint32_t w) {
  const uint32_t t = (((w & 0x77777777u) + 0x22222222u) >> 1) & 0x66666666u;
  return t | (w & 0x88888888u);
}

// 8 mask bytes of chunk c (64 subgroups); bytes past the mask are zero.
__device__ __forceinline__ uint64_t chunk_mask(const uint8_t *mask, int64_t mbytes, int64_t c) {
  const int64_t b0 = 8 * c;
  if (b0 + 8 <= mbytes) return *(const uint64_t *)(mask + b0);
  uint64_t m = 0;
  for (int i = 0; i < 8; ++i)
    if (b0 + i < mbytes) m |= (uint64_t)mask[b0 + i] << (8 * i);
  return m;
}

__device__ __forceinline__ uint32_t load_dword_guarded(const uint8_t *base, int64_t at, int64_t total) {
  if (at + 4 <= total) return *(const uint32_t *)(base + at);
  uint32_t v = 0;
  for (int i = 0; i < 4; ++i)
    if (at + i < total) v |= (uint32_t)base[at + i] << (8 * i);
  return v;
}

// Per-lane plan entry of one (chunk, lane group): byte selectors (one per
// subgroup slot: index 0..7 into the offset window, 0x0C = no offset) and the
// position of the window in the row's compacted offsets.
struct PlanEntry {
  uint32_t sel[4];
  int32_t pos;
  uint32_t bits;    // the 16 subgroup bits of the lane group
};

__device__ __forceinline__ PlanEntry make_entry(uint32_t m16, int32_t pos) {
  PlanEntry e;
  uint32_t j = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int s = 4 * q + b;
      const uint32_t on = (m16 >> s) & 1u;
      w |= (on ? j : 0x0Cu) << (8 * b);
      j += on;
    }
    e.sel[q] = w;
  }
  e.pos = pos;
  e.bits = m16;
  return e;
}

struct WChunk {
  uint32_t c[8];    // 64 E2M1 codes
  uint32_t s;       // 4 E4M3 group scales
  uint32_t o[3];    // offset dwords covering the lane's offset window
};

// Weight codes and scales of one lane for chunk c (elements e0 .. e0+63).
template <bool FAST>
__device__ __forceinline__ void load_codes(const uint8_t *crow, const uint8_t *srow, int64_t K, int64_t e0,
                                           bool live, WChunk &w) {
  if (FAST) {
    if (live && e0 < K) {   // K % 64 == 0: the lane's 64 elements are all in range
      const uint4 a = *(const uint4 *)(crow + (e0 >> 1));
      const uint4 b = *(const uint4 *)(crow + (e0 >> 1) + 16);
      w.c[0] = a.x; w.c[1] = a.y; w.c[2] = a.z; w.c[3] = a.w;
      w.c[4] = b.x; w.c[5] = b.y; w.c[6] = b.z; w.c[7] = b.w;
      w.s = *(const uint32_t *)(srow + (e0 >> 4));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w.c[i] = 0;
      w.s = 0;
    }
  } else {
    w.s = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t e = e0 + 16 * g;
      if (live && e < K) {
        const uint2 v = *(const uint2 *)(crow + (e >> 1));
        w.c[2 * g] = v.x;
        w.c[2 * g + 1] = v.y;
        w.s |= (uint32_t)srow[e >> 4] << (8 * g);
      } else {
        w.c[2 * g] = 0;
        w.c[2 * g + 1] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Activation decode: fp16 B_A * (q + delta_A) of 8 consecutive elements
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 act_decode8(const LinearArgs &a, int64_t tok, int64_t k0, bool refine) {
  if (k0 >= a.k) return make_uint4(0, 0, 0, 0);
  const uint32_t cw = *(const uint32_t *)(a.x_codes + tok * (a.k >> 1) + (k0 >> 1));
  half2v h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0);
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1);
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2);
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3);
  if (refine) {
    const uint32_t ob = *(const uint16_t *)(a.x_offsets + tok * (a.k >> 2) + (k0 >> 2));
    const uint2 d0 = delta_words(ob & 0xFFu), d1 = delta_words(ob >> 8);
    h[0] += as_h2(d0.x);
    h[1] += as_h2(d0.y);
    h[2] += as_h2(d1.x);
    h[3] += as_h2(d1.y);
  }
  const _Float16 B = (_Float16)e4m3_value(a.x_scales[tok * (a.k >> 4) + (k0 >> 4)]);
  const half2v b2 = half2v{B, B};
  return make_uint4(as_u(h[0] * b2), as_u(h[1] * b2), as_u(h[2] * b2), as_u(h[3] * b2));
}

// fp16 panel of the activations for the workspace path: xh[b][kpad],
// zero-padded past k. One thread per 8 elements.
__global__ __launch_bounds__(256) void act_dequant_kernel(LinearArgs a) {
  const int64_t per_row = a.kpad / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.b * per_row) return;
  const int64_t row = idx / per_row;
  const int64_t k0 = (idx - row * per_row) * 8;
  const bool refine = run_level(a) == 6 && a.x_offsets != nullptr;
  *(uint4 *)(a.xh + row * a.kpad + k0) = act_decode8(a, row, k0, refine);
}

// ---------------------------------------------------------------------------
// Streaming GEMV, up to 16 tokens per launch
// ---------------------------------------------------------------------------
//
// Dynamic LDS layout: [delta table 256 x 8 B][activations B x kp fp16 (XLDS)
// or nothing], the reduction buffer W x 64 x 16 B aliasing the activations
// after the main loop.
template <bool XLDS, bool FAST>
__global__ __launch_bounds__(1024) void gemv_stream_kernel(LinearArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint2 *lut = (uint2 *)lds;
  _Float16 *xs = (_Float16 *)(lds + 256 * sizeof(uint2));
  float4v *red = (float4v *)(lds + 256 * sizeof(uint2));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int64_t K = a.k;
  const int64_t nch = (K + kCh - 1) / kCh;
  const int64_t kp = nch * kCh;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int L = run_level(a);
  const bool refine_w = (L == 6) && a.w_mask != nullptr && a.n_refined > 0 && a.w_offsets != nullptr;
  const bool refine_x = (L == 6) && a.x_offsets != nullptr;

  const int64_t row = n0 + r;
  const bool row_ok = row < a.n;
  const uint8_t *crow = a.w_codes + (row_ok ? row : 0) * (K >> 1);
  const uint8_t *srow = a.w_scales + (row_ok ? row : 0) * (K >> 4);
  const int64_t obase = (row_ok ? row : 0) * (int64_t)a.n_refined;
  const int64_t ototal = a.n * (int64_t)a.n_refined;
  const int64_t mbytes = (K + 31) >> 5;

  const int64_t c0 = (nch * wave) / nw;
  const int64_t c1 = (nch * (wave + 1)) / nw;

  // 1. first weight loads
  WChunk buf[kInflight];
#pragma unroll
  for (int u = 0; u < kInflight; ++u) {
    const int64_t c = c0 + u;
    load_codes<FAST>(crow, srow, K, c * kCh + 64 * ks, row_ok && c < c1, buf[u]);
    buf[u].o[0] = buf[u].o[1] = buf[u].o[2] = 0;
  }

  // 2. offset plan of this wavefront (lane = 4 * chunk + lane group)
  PlanEntry pe{};
  int64_t pbase = c0;   // first chunk of the current plan
  int32_t pdone = 0;    // refined subgroups before chunk pbase
  if (refine_w && c0 < c1) {
    int32_t before = 0;
    for (int64_t i = lane; i < 8 * c0 && i < mbytes; i += 64) before += __popc((uint32_t)a.w_mask[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
    pdone = before;
  }
  auto build_plan = [&](int64_t cbase) {
    const int64_t ce = cbase + (lane >> 2);
    const uint64_t m64 = (ce < c1) ? chunk_mask(a.w_mask, mbytes, ce) : 0ull;
    const uint32_t m16 = (uint32_t)(m64 >> (16 * (lane & 3))) & 0xFFFFu;
    const int32_t cnt = __popc(m16);
    int32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    pe = make_entry(m16, pdone + incl - cnt);
    pdone += __shfl(incl, 63, 64);
  };
  auto offsets_load = [&](int64_t c, WChunk &w) {
    const int src = 4 * (int)(c - pbase) + ks;
    const int32_t pos = __shfl(pe.pos, src, 64);
    const uint32_t bits = __shfl(pe.bits, src, 64);
    if (row_ok && bits != 0u) {
      const int64_t at = obase + pos;
      const int64_t al = at & ~(int64_t)3;
      w.o[0] = load_dword_guarded(a.w_offsets, al, ototal);
      w.o[1] = load_dword_guarded(a.w_offsets, al + 4, ototal);
      w.o[2] = load_dword_guarded(a.w_offsets, al + 8, ototal);
    }
  };
  if (refine_w && c0 < c1) {
    build_plan(pbase);
#pragma unroll
    for (int u = 0; u < kInflight; ++u)
      if (c0 + u < c1) offsets_load(c0 + u, buf[u]);
  }

  // 3. block prologue: delta table, LDS activations
  if (refine_w) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) lut[i] = delta_words((uint32_t)i);
  }
  if (XLDS) {
    const int64_t per_row = kp / 8;
    for (int64_t i = threadIdx.x; i < a.b * per_row; i += blockDim.x) {
      const int64_t t = i / per_row;
      const int64_t k0 = (i - t * per_row) * 8;
      *(uint4 *)(xs + t * kp + k0) = act_decode8(a, t, k0, refine_x);
    }
  }
  __syncthreads();

  // 4. main loop
  float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
  const bool tok_ok = r < a.b;
  const _Float16 *xrow = XLDS ? xs + (tok_ok ? r : 0) * kp : a.xh + (tok_ok ? r : 0) * a.kpad;

  auto process = [&](int64_t c, const WChunk &w) {
    const int64_t e0 = c * kCh + 64 * ks;
    const half2v s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.s, 1.0f, false);
    const half2v s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.s, 1.0f, true);
    uint32_t E[4] = {0, 0, 0, 0};
    uint32_t any = 0;
    if (refine_w) {
      const int src = 4 * (int)(c - pbase) + ks;
      const uint32_t b16 = __shfl(pe.bits, src, 64);
      any = b16 | __shfl_xor(b16, 16, 64);
      any |= __shfl_xor(any, 32, 64);
      any = __builtin_amdgcn_readfirstlane(any);
      if (any) {
        const int32_t pos = __shfl(pe.pos, src, 64);
        const uint32_t sh = (uint32_t)((obase + pos) & 3);
        const uint32_t lo = __builtin_amdgcn_alignbyte(w.o[1], w.o[0], sh);
        const uint32_t hi = __builtin_amdgcn_alignbyte(w.o[2], w.o[1], sh);
#pragma unroll
        for (int q = 0; q < 4; ++q) E[q] = __builtin_amdgcn_perm(hi, lo, __shfl(pe.sel[q], src, 64));
      }
    }
    // two halves of 32 elements: 4 MFMAs each
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      half8v xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = tok_ok ? *(const half8v *)(xrow + e0 + 32 * hf + 8 * i) : half8v{0, 0, 0, 0, 0, 0, 0, 0};
      half2v h[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t cw = (L == 2) ? autofp2_remap(w.c[4 * hf + i]) : w.c[4 * hf + i];
        h[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0);
        h[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1);
        h[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2);
        h[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3);
      }
      if (refine_w) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int s = 8 * hf + t;
          if (any & (1u << s)) {
            const uint32_t byte = (E[s >> 2] >> (8 * (s & 3))) & 0xFFu;
            const uint2 d = lut[byte];
            h[2 * t] += as_h2(d.x);
            h[2 * t + 1] += as_h2(d.y);
          }
        }
      }
      const _Float16 b0 = hf ? s23[0] : s01[0];
      const _Float16 b1 = hf ? s23[1] : s01[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 bb = (i < 2) ? b0 : b1;
        const half2v b2 = half2v{bb, bb};
        const half2v p0 = h[4 * i] * b2, p1 = h[4 * i + 1] * b2, p2 = h[4 * i + 2] * b2, p3 = h[4 * i + 3] * b2;
        const half8v wv = half8v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv[i], acc, 0, 0, 0);
      }
    }
  };

  for (int64_t g = c0; g < c1; g += kInflight) {
    if (refine_w && g - pbase >= kPlanChunks) {
      // next plan round (kPlanChunks is a multiple of kInflight, so rounds
      // start at a group): the buffered chunks g .. g+kInflight-1 still lack
      // their offsets
      pbase = g;
      build_plan(pbase);
#pragma unroll
      for (int u = 0; u < kInflight; ++u)
        if (g + u < c1) offsets_load(g + u, buf[u]);
    }
#pragma unroll
    for (int u = 0; u < kInflight; ++u) {
      const int64_t c = g + u;
      if (c < c1) {
        process(c, buf[u]);
        const int64_t cn = c + kInflight;
        if (cn < c1) {
          load_codes<FAST>(crow, srow, K, cn * kCh + 64 * ks, row_ok, buf[u]);
          buf[u].o[0] = buf[u].o[1] = buf[u].o[2] = 0;
          if (refine_w && cn - pbase < kPlanChunks) offsets_load(cn, buf[u]);
        }
      }
    }
  }

  // 5. sum the wavefront tiles and store
  __syncthreads();
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float4v s = red[lane];
  for (int w = 1; w < nw; ++w) s += red[w * 64 + lane];
  if (!tok_ok) return;
  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
  const int64_t nb = n0 + 4 * ks;
  const int64_t tok = r;
  if (a.y_dtype == AUTOFP_BF16) {
    uint16_t *y = (uint16_t *)a.y + tok * a.n;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (nb + v < a.n) y[nb + v] = f32_to_bf16_rne(s[v] * scale);
  } else {
    float *y = (float *)a.y + tok * a.n;
    if (nb + 3 < a.n && (a.n & 3) == 0) {
      *(float4v *)(y + nb) = s * scale;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (nb + v < a.n) y[nb + v] = s[v] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// GEMV for 17..64 tokens: activations from the fp16 panel
// ---------------------------------------------------------------------------

struct WRow {
  const uint8_t *codes, *scales, *offs;
  int64_t K;
  bool ok, k32;
};

__device__ __forceinline__ void load_w(const WRow &w, int64_t ke, bool live, uint4 &cw, uint32_t &sw) {
  cw = make_uint4(0, 0, 0, 0);
  sw = 0;
  if (!(live && w.ok && ke < w.K)) return;
  if (w.k32) {
    cw = *(const uint4 *)(w.codes + (ke >> 1));
    sw = *(const uint16_t *)(w.scales + (ke >> 4));
  } else {
    const uint2 lo = *(const uint2 *)(w.codes + (ke >> 1));
    cw.x = lo.x;
    cw.y = lo.y;
    sw = w.scales[ke >> 4];
    if (ke + 16 < w.K) {
      const uint2 hi = *(const uint2 *)(w.codes + (ke >> 1) + 8);
      cw.z = hi.x;
      cw.w = hi.y;
      sw |= (uint32_t)w.scales[(ke >> 4) + 1] << 8;
    }
  }
}

// Decoded weight operand B_W * (q + delta) (or B_W * Q at level 2) of one
// lane's 32 elements; `pre` tracks the compacted-offset position of the row.
__device__ __forceinline__ void decode_w(const LinearArgs &a, const WRow &w, int L, bool refine_w,
                                         int64_t c, int ks, uint4 cw, uint32_t sw, int32_t &pre,
                                         half8v h[4]) {
  uint32_t w4[4] = {cw.x, cw.y, cw.z, cw.w};
  if (L == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w4[i] = autofp2_remap(w4[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = fp4x8_to_half8(w4[i]);
  if (refine_w) {
    const int64_t mbytes = (w.K + 31) >> 5;
    uint32_t md;
    if (4 * c + 3 < mbytes) {
      md = *(const uint32_t *)(a.w_mask + 4 * c);
    } else {
      md = 0;
      for (int j = 0; j < 4 && 4 * c + j < mbytes; ++j) md |= (uint32_t)a.w_mask[4 * c + j] << (8 * j);
    }
    uint32_t mb = (md >> (8 * ks)) & 0xFFu;
    int32_t pos = pre + __popc(md & ((1u << (8 * ks)) - 1u));
    pre += __popc(md);
    if (!w.ok) mb = 0;
    while (mb) {
      const int sg = __ffs(mb) - 1;
      mb &= mb - 1;
      half2v lo, hi;
      offsets_to_half4(w.offs[pos++], lo, hi);
      const half8v dl = (sg & 1) ? half8v{0, 0, 0, 0, lo[0], lo[1], hi[0], hi[1]}
                                 : half8v{lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
      switch (sg >> 1) {
        case 0: h[0] += dl; break;
        case 1: h[1] += dl; break;
        case 2: h[2] += dl; break;
        default: h[3] += dl; break;
      }
    }
  }
  const _Float16 b0 = (_Float16)e4m3_value(sw & 0xFFu);
  const _Float16 b1 = (_Float16)e4m3_value(sw >> 8);
  h[0] *= b0;
  h[1] *= b0;
  h[2] *= b1;
  h[3] *= b1;
}

// Refined subgroups of the row before chunk c0 (chunks before c0 are
// complete, so their four mask bytes exist).
__device__ __forceinline__ int32_t w_prefix(const LinearArgs &a, int64_t c0) {
  int32_t pre = 0;
  for (int64_t m = 0; m < c0; ++m) pre += __popc(*(const uint32_t *)(a.w_mask + 4 * m));
  return pre;
}

template <int TT, int U>
__global__ __launch_bounds__(256) void gemv_panel_kernel(LinearArgs a) {
  __shared__ float4v red[4][TT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int64_t K = a.k;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int L = run_level(a);
  const bool refine_w = (L == 6) && a.w_mask != nullptr && a.w_offsets != nullptr;

  WRow w;
  const int64_t row = n0 + r;
  w.ok = row < a.n;
  w.K = K;
  w.k32 = (K & 31) == 0;
  w.codes = a.w_codes + (w.ok ? row : 0) * (K >> 1);
  w.scales = a.w_scales + (w.ok ? row : 0) * (K >> 4);
  w.offs = refine_w ? a.w_offsets + (w.ok ? row : 0) * (int64_t)a.n_refined : nullptr;

  const int64_t nch = (K + 127) >> 7;
  const int64_t per = (nch + 3) >> 2;
  const int64_t c0 = wave * per;
  const int64_t c1 = (c0 + per < nch) ? c0 + per : nch;
  int32_t pre = (refine_w && c0 < c1) ? w_prefix(a, c0) : 0;

  float4v acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t cb = c0; cb < c1; cb += U) {
    uint4 cw[U];
    uint32_t sw[U];
    half8v xv[U][TT][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      const int64_t ke = (c << 7) + (ks << 5);
      load_w(w, ke, c < c1, cw[u], sw[u]);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int64_t tok = 16 * t + r;
        const bool tok_ok = (c < c1) && tok < a.b;
        const half8v *src = (const half8v *)(a.xh + (tok_ok ? tok : 0) * a.kpad + (c < c1 ? ke : 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[u][t][i] = tok_ok ? src[i] : half8v{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      if (c >= c1) break;
      half8v h[4];
      decode_w(a, w, L, refine_w, c, ks, cw[u], sw[u], pre, h);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h[i], xv[u][t][i], acc[t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < TT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float4v s = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
    const int64_t tok = 16 * t + r;
    if (tok >= a.b) continue;
    const int64_t nb = n0 + 4 * ks;
    if (a.y_dtype == AUTOFP_BF16) {
      uint16_t *y = (uint16_t *)a.y + tok * a.n;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (nb + v < a.n) y[nb + v] = f32_to_bf16_rne(s[v] * scale);
    } else {
      float *y = (float *)a.y + tok * a.n;
      if (nb + 3 < a.n && (a.n & 3) == 0) {
        *(float4v *)(y + nb) = s * scale;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (nb + v < a.n) y[nb + v] = s[v] * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch configuration of the streaming kernel
// ---------------------------------------------------------------------------

struct StreamCfg {
  int waves;
  bool xlds;
  bool fast;
  size_t lds;
};

int max_lds_per_block() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
      v = 65536;
    cached[dev] = v;
  }
  return cached[dev];
}

StreamCfg stream_cfg(const LinearArgs &a) {
  StreamCfg c{};
  const int64_t nch = (a.k + kCh - 1) / kCh;
  const int64_t blocks = (a.n + 15) / 16;
  int64_t w = (4096 + blocks - 1) / blocks;   // aim at 4096 wavefronts in the grid
  int p = 1;
  while (p < w && p < kMaxWaves) p <<= 1;
  while (p > 1 && p > nch) p >>= 1;
  if (a.waves > 0) p = a.waves;
  c.waves = p;
  c.fast = (a.k % 64) == 0;
  const size_t lut = 256 * sizeof(uint2);
  const size_t red = (size_t)p * 64 * sizeof(float4v);
  const size_t xs = (size_t)a.b * (size_t)(nch * kCh) * sizeof(_Float16);
  const size_t budget = max_lds_per_block() < 65536 ? (size_t)max_lds_per_block() : 65536;
  c.xlds = lut + (xs > red ? xs : red) <= budget;
  c.lds = lut + (c.xlds ? (xs > red ? xs : red) : red);
  return c;
}

}  // namespace

int64_t xh_kpad(int64_t k) { return round_up(k, kCh); }

bool gemv_needs_panel(const LinearArgs &a) {
  if (a.b > 16) return true;
  return !stream_cfg(a).xlds;
}

hipError_t launch_act_dequant(const LinearArgs &a, hipStream_t s) {
  const int64_t threads = a.b * (a.kpad / 8);
  hipLaunchKernelGGL(act_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const LinearArgs &a0, hipStream_t s) {
  if (a0.b <= 16) {
    const StreamCfg c = stream_cfg(a0);
    const dim3 grid((unsigned)((a0.n + 15) / 16)), block((unsigned)(64 * c.waves));
    if (c.xlds) {
      if (c.fast) hipLaunchKernelGGL((gemv_stream_kernel<true, true>), grid, block, c.lds, s, a0);
      else hipLaunchKernelGGL((gemv_stream_kernel<true, false>), grid, block, c.lds, s, a0);
    } else {
      if (c.fast) hipLaunchKernelGGL((gemv_stream_kernel<false, true>), grid, block, c.lds, s, a0);
      else hipLaunchKernelGGL((gemv_stream_kernel<false, false>), grid, block, c.lds, s, a0);
    }
    return hipGetLastError();
  }
  // slices of at most 64 tokens
  for (int64_t t0 = 0; t0 < a0.b; t0 += 64) {
    LinearArgs a = a0;
    a.b = (a0.b - t0) < 64 ? (a0.b - t0) : 64;
    a.xh = a0.xh + t0 * a0.kpad;
    a.x_codes = a0.x_codes + t0 * (a0.k / 2);
    a.x_scales = a0.x_scales + t0 * (a0.k / 16);
    a.x_offsets = a0.x_offsets ? a0.x_offsets + t0 * (a0.k / 4) : nullptr;
    a.y = (char *)a0.y + t0 * a0.n * (a0.y_dtype == AUTOFP_BF16 ? 2 : 4);
    const dim3 grid((unsigned)((a.n + 15) / 16));
    if (a.b <= 16) {
      hipLaunchKernelGGL((gemv_panel_kernel<1, 4>), grid, dim3(256), 0, s, a);
    } else if (a.b <= 32) {
      hipLaunchKernelGGL((gemv_panel_kernel<2, 4>), grid, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((gemv_panel_kernel<4, 2>), grid, dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace afp
