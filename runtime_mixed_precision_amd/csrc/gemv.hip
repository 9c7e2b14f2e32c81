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
// 4 or 8 chunks of loads in flight. The activation operand comes from an
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

#include <atomic>

#include "afp_act.h"
#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
typedef int32_t i32x8v __attribute__((ext_vector_type(8)));

constexpr int kCh = 256;         // K elements per chunk
constexpr int kGroup = 4;        // chunks per scale load group
constexpr int kMaxWaves = 16;    // wavefronts per block (1024 threads)
constexpr int kPlanChunks = 16;  // chunks per wavefront covered by its offset plan
constexpr int kProMask = 2;      // weight-mask dwords per thread loaded by the block prologue

__device__ __forceinline__ int run_level(const LinearArgs &a) {
  return a.bits_dev ? *a.bits_dev : a.bits;
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

// Per-lane plan entry of one (chunk, lane group): byte selectors (one per
// subgroup slot: index 0..7 into the offset window, 0x0C = no offset) and the
// position of the window in the row's compacted offsets.
struct PlanEntry {
  uint32_t sel[4];
  int32_t pos;
};
constexpr int kPlanBytesPerWave = 64 * 20;   // 64 entries: selectors (16 B) and position (4 B)

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
  return e;
}

struct WChunk {
  uint32_t c[8];    // 64 E2M1 codes
  uint32_t s;       // 4 E4M3 group scales
  uint32_t o[3];    // offset dwords covering the lane's offset window
};

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

// The same decode from already loaded bytes: 8 codes, their group scale byte
// and (refine) the two offset bytes of their subgroups.
__device__ __forceinline__ uint4 act_decode8_vals(uint32_t cw, uint32_t sbyte, uint32_t ob, bool refine) {
  half2v h[4];
  h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0);
  h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1);
  h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2);
  h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3);
  if (refine) {
    const uint2 d0 = delta_words(ob & 0xFFu), d1 = delta_words((ob >> 8) & 0xFFu);
    h[0] += as_h2(d0.x);
    h[1] += as_h2(d0.y);
    h[2] += as_h2(d1.x);
    h[3] += as_h2(d1.y);
  }
  const _Float16 B = (_Float16)e4m3_value(sbyte & 0xFFu);
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
  const int level = run_level(a);
  if (a.fmt != AUTOFP_FMT_AUTOFP6) {
    const bool refine = (level == 6 || (level == 8 && a.fmt == AUTOFP_FMT_AUTOFP8)) && a.x_offsets != nullptr;
    *(uint4 *)(a.xh + row * a.kpad + k0) = act_decode8_fmt(a, row, k0, refine, level);
    return;
  }
  const bool refine = level == 6 && a.x_offsets != nullptr;
  *(uint4 *)(a.xh + row * a.kpad + k0) = act_decode8(a, row, k0, refine);
}

// ---------------------------------------------------------------------------
// Streaming GEMV, up to 16 tokens per launch
// ---------------------------------------------------------------------------
//
// Dynamic LDS layout: [delta table 256 x 8 B][weight-mask copy][XLDS:
// activations B x kp fp16 at a row pitch of kp + 8 (16 bytes of padding put
// the rows of different tokens on different LDS banks), then a 128-byte zero
// row read by the lanes of absent tokens][level 6: each wavefront's offset
// plan, 64 x 16 B selectors then 64 x 4 B positions]; the
// reduction buffer W x 64 x 16 B reuses the space after the main loop.
//
// Every global read goes through a buffer resource covering the block's rows,
// so rows past the end of the weight and chunks past a wavefront's range read
// as zero (an out-of-range offset) instead of branching: each chunk issues the
// same loads, which lets the compiler keep a fixed number of chunks in flight.

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset that is always out of range
constexpr int64_t kLutBytes = 256 * 8;   // delta table

// LDS bytes of the weight-mask copy (zero-padded so 8-byte chunk reads stay inside)
__host__ __device__ __forceinline__ int64_t mask_lds_bytes(int64_t k) {
  return ((((k + 31) >> 5) + 15) / 16) * 16 + 16;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

__device__ __forceinline__ uint4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t ld_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Scheduling fence that keeps vector-memory instructions in program order
// while letting ALU, MFMA and LDS work move across it.
__device__ __forceinline__ void vmem_fence() { __builtin_amdgcn_sched_barrier(0x78F); }

// One block: RT row tiles of 16 rows x WK wavefronts per tile (RT * WK
// wavefronts, blockDim = 64 * RT * WK). Wavefront w works on tile w / WK and
// on the (w % WK)-th contiguous range of 256-element chunks of K.
// PD chunks of weight loads are kept in flight per wavefront; the block
// prologue loads up to PRO activation items (8 elements each) per thread
// ahead of the weight loads (more fall back to a plain loop).
template <int L, bool XLDS, bool FAST, int PD, int PRO>
__device__ __forceinline__ void stream_tile(const LinearArgs &a, unsigned char *lds) {
  static_assert(PD % kGroup == 0, "whole scale load groups");
  constexpr int NG = PD / kGroup;   // scale load groups in flight
  constexpr bool REF = (L == 6);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int WK = a.wk;
  const int tile = wave / WK;
  const int kw = wave - tile * WK;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int64_t K = a.k;
  const int64_t nch = (K + kCh - 1) / kCh;
  const int64_t kp = nch * kCh;
  const int64_t xpitch = kp + 8;   // LDS row pitch of the activations (halves)
  const int64_t n0 = ((int64_t)blockIdx.x * (nw / WK) + tile) * 16;
  int64_t rows = a.n - n0;
  rows = rows < 0 ? 0 : rows > 16 ? 16 : rows;
  const int64_t R = a.n_refined;
  const bool refine_w = REF && a.w_mask != nullptr && R > 0 && a.w_offsets != nullptr;
  const bool refine_x = REF && a.x_offsets != nullptr;
  const bool tok_ok = r < a.b;
  const int64_t mbytes = (K + 31) >> 5;

  uint2 *lut = (uint2 *)lds;
  uint8_t *mlds = lds + kLutBytes;
  _Float16 *xs = (_Float16 *)(lds + kLutBytes + mask_lds_bytes(K));
  float4v *red = (float4v *)(lds + kLutBytes);
  const int64_t xs_bytes = XLDS ? (a.b * xpitch + 64) * 2 : 0;
  unsigned char *plan = lds + kLutBytes + mask_lds_bytes(K) + ((xs_bytes + 15) & ~(int64_t)15) +
                        (int64_t)wave * kPlanBytesPerWave;
  uint4 *plan_sel = (uint4 *)plan;
  int32_t *plan_pos = (int32_t *)(plan + 64 * 16);

  const int64_t nb0 = rows > 0 ? n0 : 0;   // keep resource bases inside the tensors
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w_codes + nb0 * (K >> 1), rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.w_scales + nb0 * (K >> 4), rows * (K >> 4));
  // weight offsets: the tile's rows plus the 16 padding bytes every offsets buffer carries
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(refine_w ? a.w_offsets + nb0 * R : a.w_codes, rows > 0 ? rows * R + 16 : 0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xh, XLDS ? 0 : a.b * a.kpad * 2);
  const uint32_t crow = (uint32_t)(r * (K >> 1) + 32 * ks);    // + 128 bytes per chunk
  const uint32_t orow = (uint32_t)(r * R);

  const int64_t c0 = (nch * kw) / WK;
  const int64_t c1 = (nch * (kw + 1)) / WK;

  // Weight codes and scales of chunk c. A buffer load whose range is not
  // wholly inside the resource reads as zero; chunks past the wavefront's
  // range use an out-of-range scalar offset. With K % 256 == 0 (FAST) every
  // lane's 64 elements lie inside K; otherwise each 16-element group is
  // loaded on its own.
  auto load_codes = [&](int64_t c, WChunk &w) {
    if (FAST) {
      // the chunk offset goes in the scalar offset; a chunk past the range
      // moves the lane offset out of range (the range check is made on the
      // lane offset)
      const bool live = c < c1;
      const uint32_t so = live ? (uint32_t)(c * 128) : 0u;
      const uint32_t vo = live ? crow : kOOB;
      const u32x4v lo = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)vo, (int)so, 0);
      const u32x4v hi = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(vo + 16), (int)so, 0);
      w.c[0] = lo[0]; w.c[1] = lo[1]; w.c[2] = lo[2]; w.c[3] = lo[3];
      w.c[4] = hi[0]; w.c[5] = hi[1]; w.c[6] = hi[2]; w.c[7] = hi[3];
      w.s = 0;   // scales come per load group (load_scales)
    } else {
      const int64_t e0 = c * kCh + 64 * ks;
      w.s = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t e = e0 + 16 * g;
        const bool live = c < c1 && e < K;
        const uint32_t oc = live ? (uint32_t)(r * (K >> 1) + (e >> 1)) : kOOB;
        const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)oc, 0, 0);
        w.c[2 * g] = v[0];
        w.c[2 * g + 1] = v[1];
        const uint32_t os = live ? (uint32_t)(r * (K >> 4) + (e >> 4)) : kOOB;
        w.s |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsc, (int)os, 0, 0) << (8 * g);
      }
    }
    w.o[0] = w.o[1] = w.o[2] = 0;
  };

  // Group scales (FAST): lane (r, j) loads the 16 scale bytes of row r in
  // chunk g + j - one 16-byte load per lane for a whole load group, so each
  // row's scales arrive as 64 contiguous bytes - and a 4 x 4 transpose across
  // the lane groups (v_permlane32_swap, v_permlane16_swap) leaves in register
  // u of lane (r, ks) the 4 scale bytes of its groups in chunk g + u.
  static_assert(kGroup == 4, "the scale transpose assumes 4 chunks per load group");
  uint32_t sc_ring[NG][4] = {}, sc_cur[4] = {0, 0, 0, 0};
  auto load_scales = [&](int64_t g, int slot) {
    if (!FAST) return;
    const int64_t c = g + ks;
    const uint32_t vo = (c < c1) ? (uint32_t)(r * (K >> 4) + 16 * c) : kOOB;
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rsc, (int)vo, 0, 0);
    sc_ring[slot][0] = v[0]; sc_ring[slot][1] = v[1]; sc_ring[slot][2] = v[2]; sc_ring[slot][3] = v[3];
  };
  auto transpose_scales = [&](int slot) {
    if (!FAST) return;
    const uint32_t *sn = sc_ring[slot];
    const auto a = __builtin_amdgcn_permlane32_swap(sn[0], sn[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(sn[1], sn[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    sc_cur[0] = c[0]; sc_cur[1] = c[1]; sc_cur[2] = d[0]; sc_cur[3] = d[1];
  };

  // 0. block prologue loads: the activation codes / scales / offsets and the
  //    weight mask, issued before the weight loads so that waiting for them
  //    leaves the weight loads in flight (a fixed number of loads per thread;
  //    items past the end read as zero).
  const int nthr = blockDim.x;
  const int64_t per_row = kp / 8;
  const int64_t items = XLDS ? a.b * per_row : 0;
  const int64_t mdw = refine_w ? (mbytes + 3) / 4 : 0;
  // (FAST) the first PRO items per thread go ahead of the weight loads; any
  // further items follow in rounds of 8 per thread, each round's loads issued
  // together
  const bool pro_static = FAST && mask_lds_bytes(K) <= 4 * (int64_t)kProMask * nthr;
  uint32_t pq[PRO], ps[PRO], po[PRO], pm[kProMask];
  const __amdgpu_buffer_rsrc_t rxc = make_rsrc(a.x_codes, a.b * (K >> 1));
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(a.x_scales, a.b * (K >> 4));
  const __amdgpu_buffer_rsrc_t rxo = make_rsrc(refine_x ? a.x_offsets : a.x_codes, refine_x ? a.b * (K >> 2) : 0);
  if (pro_static) {
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(refine_w ? a.w_mask : a.w_codes, refine_w ? mbytes : 0);
    // the weight-mask loads first: the mask is written to LDS before the
    // activations, so its wait leaves the activation loads in flight
    if (REF) {
#pragma unroll
      for (int j = 0; j < kProMask; ++j) {
        const uint32_t i = threadIdx.x + (uint32_t)(j * nthr);
        pm[j] = ld_b32(rm, i < (uint32_t)mdw ? 4 * i : kOOB);
      }
    }
    // Item i covers elements 8i .. 8i + 7 of the token-major activations
    // (K % 256 == 0, so no item straddles a row): code bytes 4i .. 4i + 3,
    // scale byte i / 2 and offset bytes 2i, 2i + 1.
#pragma unroll
    for (int j = 0; j < PRO; ++j) {
      const uint32_t i = threadIdx.x + (uint32_t)(j * nthr);
      const bool live = i < (uint32_t)items;
      pq[j] = ld_b32(rxc, live ? 4 * i : kOOB);
      ps[j] = __builtin_amdgcn_raw_buffer_load_b8(rxs, (int)(live ? i >> 1 : kOOB), 0, 0);
      po[j] = REF ? __builtin_amdgcn_raw_buffer_load_b16(rxo, (int)(live && refine_x ? 2 * i : kOOB), 0, 0) : 0u;
    }
    vmem_fence();
  }

  // 1. first weight loads, kept in issue order: the loop below relies on
  //    every step finding the same loads in flight, oldest buffer first. At
  //    level 6 the offsets of a chunk follow its codes, so those loads wait
  //    for the offset plan (step 3).
  WChunk buf[PD];
  if (!REF) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (u % kGroup == 0) load_scales(c0 + u, u / kGroup);
      load_codes(c0 + u, buf[u]);
      vmem_fence();
    }
  }

  // 2. block prologue in LDS: delta table, weight-mask copy, activations
  //    (+ a zero row for absent tokens)
  const int64_t mpad = mask_lds_bytes(K);
  if (refine_w) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) lut[i] = delta_words((uint32_t)i);
  }
  if (pro_static) {
    if (REF) {
#pragma unroll
      for (int j = 0; j < kProMask; ++j) {
        const uint32_t i = threadIdx.x + (uint32_t)(j * nthr);
        if (4 * i < (uint32_t)mpad) *(uint32_t *)(mlds + 4 * i) = pm[j];   // zero past the mask
      }
    }
#pragma unroll
    for (int j = 0; j < PRO; ++j) {
      const uint32_t i = threadIdx.x + (uint32_t)(j * nthr);
      if (i < (uint32_t)items) {
        const uint32_t t = i / (uint32_t)per_row;
        const uint32_t k0 = (i - t * (uint32_t)per_row) * 8;
        *(uint4 *)(xs + t * xpitch + k0) = act_decode8_vals(pq[j], ps[j], po[j], refine_x);
      }
    }
    for (int64_t base = (int64_t)PRO * nthr; base < items; base += 8 * (int64_t)nthr) {
      uint32_t q8[8], s8[8], o8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t i = (uint32_t)base + threadIdx.x + (uint32_t)(j * nthr);
        const bool live = i < (uint32_t)items;
        q8[j] = ld_b32(rxc, live ? 4 * i : kOOB);
        s8[j] = __builtin_amdgcn_raw_buffer_load_b8(rxs, (int)(live ? i >> 1 : kOOB), 0, 0);
        o8[j] = REF ? __builtin_amdgcn_raw_buffer_load_b16(rxo, (int)(live && refine_x ? 2 * i : kOOB), 0, 0) : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t i = (uint32_t)base + threadIdx.x + (uint32_t)(j * nthr);
        if (i < (uint32_t)items) {
          const uint32_t t = i / (uint32_t)per_row;
          const uint32_t k0 = (i - t * (uint32_t)per_row) * 8;
          *(uint4 *)(xs + t * xpitch + k0) = act_decode8_vals(q8[j], s8[j], o8[j], refine_x);
        }
      }
    }
  } else {
    if (refine_w) {
      for (int64_t i = threadIdx.x; i < mpad; i += blockDim.x) mlds[i] = i < mbytes ? a.w_mask[i] : 0;
    }
    if (XLDS) {
      for (int64_t i = threadIdx.x; i < items; i += blockDim.x) {
        const int64_t t = i / per_row;
        const int64_t k0 = (i - t * per_row) * 8;
        *(uint4 *)(xs + t * xpitch + k0) = act_decode8(a, t, k0, refine_x);
      }
    }
  }
  if (XLDS && threadIdx.x < 8) *(uint4 *)(xs + a.b * xpitch + 8 * threadIdx.x) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // 3. offset plan of this wavefront (lane = 4 * chunk + lane group), from
  //    the LDS mask copy, and the first offset loads
  const int64_t pbase = c0;
  auto build_plan = [&](int32_t pdone) {
    const int64_t ce = pbase + (lane >> 2);
    const uint64_t m64 = (ce < c1) ? *(const uint64_t *)(mlds + 8 * ce) : 0ull;
    const uint32_t m16 = (uint32_t)(m64 >> (16 * (lane & 3))) & 0xFFFFu;
    const int32_t cnt = __popc(m16);
    int32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const PlanEntry pe = make_entry(m16, pdone + incl - cnt);
    plan_sel[lane] = make_uint4(pe.sel[0], pe.sel[1], pe.sel[2], pe.sel[3]);
    plan_pos[lane] = pe.pos;
  };
  // the 12 aligned bytes holding the lane's (at most 8) offset bytes of chunk c
  auto offsets_load = [&](int64_t c, WChunk &w) {
    const bool live = refine_w && c < c1;
    const int32_t pos = live ? plan_pos[4 * (int)(c - pbase) + ks] : 0;
    const uint32_t al = live ? ((orow + (uint32_t)pos) & ~3u) : kOOB;
    const u32x3v v = __builtin_amdgcn_raw_buffer_load_b96(ro, (int)al, 0, 0);
    w.o[0] = v[0];
    w.o[1] = v[1];
    w.o[2] = v[2];
  };
  if (refine_w) {
    int32_t before = 0;
    for (int64_t i = lane; i < 8 * c0; i += 64) before += __popc((uint32_t)mlds[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
    build_plan(before);
  }
  if (REF) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (u % kGroup == 0) load_scales(c0 + u, u / kGroup);
      load_codes(c0 + u, buf[u]);
      offsets_load(c0 + u, buf[u]);
      vmem_fence();
    }
  }

  // 4. main loop
  float4v acc0 = float4v{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  const _Float16 *xrow = xs + (tok_ok ? r * xpitch : 0) + 64 * ks;
  const _Float16 *xzero = xs + a.b * xpitch;
  const uint32_t xoff_row = (uint32_t)(r * a.kpad * 2 + 128 * ks);

  auto process = [&](int64_t c, const WChunk &w, uint32_t sc) {
    uint32_t cw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cw[i] = (L == 2) ? autofp2_remap(w.c[i]) : w.c[i];
    const half2v s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
    const half2v s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true);

    uint32_t wlo = 0, whi = 0;
    uint4 sel = make_uint4(0, 0, 0, 0);
    if (refine_w) {
      const int ent = 4 * (int)(c - pbase) + ks;
      sel = plan_sel[ent];
      const uint32_t sh = (orow + (uint32_t)plan_pos[ent]) & 3u;
      wlo = __builtin_amdgcn_alignbyte(w.o[1], w.o[0], sh);
      whi = __builtin_amdgcn_alignbyte(w.o[2], w.o[1], sh);
    }

    const _Float16 *xp = tok_ok ? xrow + c * kCh : xzero;
    const uint32_t xo = tok_ok ? xoff_row + (uint32_t)(c * kCh * 2) : kOOB;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      half8v xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (XLDS) {
          xv[i] = *(const half8v *)(xp + 32 * hf + 8 * i);
        } else {
          const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xo + 64 * hf + 16 * i), 0, 0);
          xv[i] = __builtin_bit_cast(half8v, v);
        }
      }
      half2v h[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = cw[4 * hf + i];
        h[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0);
        h[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1);
        h[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2);
        h[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3);
      }
      if (refine_w) {
        // one offset byte per subgroup slot of this half (0 where not refined)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const uint32_t sq = (2 * hf + qq == 0) ? sel.x : (2 * hf + qq == 1) ? sel.y : (2 * hf + qq == 2) ? sel.z : sel.w;
          const uint32_t E = __builtin_amdgcn_perm(whi, wlo, sq);
          uint2 d[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) d[t] = lut[(E >> (8 * t)) & 0xFFu];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            h[8 * qq + 2 * t] += as_h2(d[t].x);
            h[8 * qq + 2 * t + 1] += as_h2(d[t].y);
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
        if (i & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv[i], acc1, 0, 0, 0);
        else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, xv[i], acc0, 0, 0, 0);
      }
    }
  };

  // PD buffered chunks per step, each processed and then refilled with the
  // chunk PD ahead, so PD - 1 chunks stay in flight while one is computed;
  // each scale load group is loaded with the first chunk of its group.
  for (int64_t g = c0; g < c1; g += PD) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      transpose_scales(j);
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int b = kGroup * j + u;
        const int64_t c = g + b;
        if (c < c1) process(c, buf[b], FAST ? sc_cur[u] : buf[b].s);
        vmem_fence();
        if (u == 0) load_scales(c + PD, j);
        load_codes(c + PD, buf[b]);
        if (REF) offsets_load(c + PD, buf[b]);   // unconditional loads: uniform waits
        vmem_fence();
      }
    }
  }

  // 5. sum the K-split tiles of each row tile and store
  const float4v acc = acc0 + acc1;
  __syncthreads();
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (kw != 0 || rows == 0) return;
  float4v s = red[wave * 64 + lane];
  for (int w = 1; w < WK; ++w) s += red[(wave + w) * 64 + lane];
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

// PD = 4: blocks of up to 1024 threads, 128 VGPRs; PD = 8: up to 512 threads,
// 256 VGPRs (two wavefronts per SIMD).
template <bool XLDS, bool FAST, int PD, int PRO>
__global__ __launch_bounds__(PD == 8 ? 512 : 1024) void gemv_stream_kernel(LinearArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int L = run_level(a);
  if (L == 6) stream_tile<6, XLDS, FAST, PD, PRO>(a, lds);
  else if (L == 2) stream_tile<2, XLDS, FAST, PD, PRO>(a, lds);
  else stream_tile<4, XLDS, FAST, PD, PRO>(a, lds);
}

// ---------------------------------------------------------------------------
// One-token GEMV on the fp4 matrix cores (levels 2 and 4)
// ---------------------------------------------------------------------------
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in E2M1 (scales 2^0)
// multiplies a 16 x 128 block by a 128 x 16 block exactly: every product is
// a multiple of 1/4 of magnitude at most 36. The weight codes enter unchanged
// as the B operand (column j = weight row j; lane l holds column l % 16 and
// the 32 elements 32 * (l / 16) .. + 31 of the MFMA's K range, low nibble
// first). The A operand is the activation laid out block-diagonally: row s
// holds the 16 codes of one 16-element group and zeros elsewhere, so
// D[s][j] is the exact dot product of that group of the activation with
// weight row j. The E4M3 group scales of both operands are applied to D in
// fp32, so no element is converted: per 256-element chunk a lane does two
// MFMAs and 16 scale multiply-adds instead of 32 fp4 -> fp16 conversions.
//
// A lane (row r = l % 16, lane group q = l / 16) loads, per chunk, the same
// 32 code bytes as the streaming kernel: elements 64q .. 64q + 63, the first
// half for MFMA h = 0 and the second for h = 1. MFMA h thus sees, in lane
// group q, the groups 4q + 2h and 4q + 2h + 1 of the chunk; A row s < 8 is
// the group 4 * (s / 2) + 2h + s % 2. Output lane (r, q) holds rows 4q .. 4q+3
// of D, i.e. for q < 2 the groups 8q + {0, 1, 4, 5} + 2h of weight row r.
constexpr int kFp4Chunks = 16;                          // chunks per wavefront at most
constexpr int kFp4Pitch = kFp4Chunks * 16 + 16;            // LDS row pitch of the weight scales
constexpr int kFp4Depth = 8;                               // chunks of code loads in flight
constexpr int kFp4Depth6 = 4;                              // level 6 (offset windows too)

// Wavefront-private LDS of the matrix-core GEMV for up to BT tokens: weight
// scales [16 rows][16 chunks][16 B] at a row pitch of 272 B (the 16 rows'
// reads then cover all 64 banks once); the activation codes [BT][cap][128 B]
// and scales as fp32 [BT][cap][16]; then at level 6 the activation offsets as
// E2M1 d/2 codes [BT][cap][128 B], the offset plan and the offset-byte table,
// or at levels 2 and 4 a 2 KB slot where each chunk's codes change lane
// layout. cap (chunks per wavefront) keeps BT * cap <= 32 above one token.
template <int BT>
struct Fp4Lay {
  static constexpr int cap = BT == 1 ? kFp4Chunks : 32 / BT;
  static constexpr int tc = BT * cap;
  static constexpr int xs = 16 * kFp4Pitch;
  static constexpr int sx = xs + tc * 128;
  static constexpr int dx = sx + tc * 64;
  static constexpr int plan = dx + tc * 128;
  static constexpr int lut = plan + kPlanBytesPerWave;
  static constexpr int bytes4 = dx + 2048;
  static constexpr int bytes6 = lut + 512;
};

// Four 2-bit offsets d (two's complement, element e in bits 2e+1:2e) as four
// E2M1 codes of d/2 in the nibbles of a 16-bit value: +1 -> 0.5 (0001),
// 0 -> 0, -1 -> -0.5 (1001), -2 -> -1 (1010). Two bytes at once: byte j of
// v (j = 0, 1) -> bits 16j .. 16j + 15.
__device__ __forceinline__ uint32_t offsets_to_e2m1(uint32_t v) {
  uint32_t t = v & 0xFFFFu;
  t = (t | (t << 8)) & 0x00FF00FFu;
  t = (t | (t << 4)) & 0x0F0F0F0Fu;
  t = (t | (t << 2)) & 0x33333333u;
  const uint32_t b0 = t & 0x11111111u, b1 = (t >> 1) & 0x11111111u;
  return b0 | (b1 << 3) | ((b1 & ~b0) << 1);
}

// Up to BT tokens: each MFMA's 16 A rows hold 8 group slots of two tokens
// (levels 2 and 4: tokens 2m and 2m + 1) or of one token's codes and its
// offsets d/2 (level 6: token m), so M = ceil(BT / 2) or BT MFMAs per
// half-chunk reuse one weight operand.
template <int L, int PD, bool ROWS, int BT>
__device__ __forceinline__ void fp4_tile(const LinearArgs &a, unsigned char *lds) {
  constexpr bool REF = (L == 6);
  constexpr bool P3 = ROWS && !REF;
  constexpr int M = REF ? BT : (BT + 1) / 2;
  typedef Fp4Lay<BT> Lay;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int WK = a.wk;
  const int tile = wave / WK;
  const int kw = wave - tile * WK;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int B = (int)a.b;
  const int64_t K = a.k;
  const int64_t nch = K / kCh;
  const int64_t n0 = ((int64_t)blockIdx.x * (nw / WK) + tile) * 16;
  int64_t rows = a.n - n0;
  rows = rows < 0 ? 0 : rows > 16 ? 16 : rows;
  const int64_t nb0 = rows > 0 ? n0 : 0;
  const int64_t c0 = (nch * kw) / WK;
  const int64_t c1 = (nch * (kw + 1)) / WK;
  const int len = (int)(c1 - c0);   // at most Lay::cap
  const int64_t R = a.n_refined;
  const bool refine_w = REF && a.w_mask != nullptr && R > 0 && a.w_offsets != nullptr;
  const bool refine_x = REF && a.x_offsets != nullptr;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.w_codes + nb0 * (K >> 1), rows * (K >> 1));
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.w_scales + nb0 * (K >> 4), rows * (K >> 4));
  // weight offsets: the tile's rows plus the 16 padding bytes every offsets buffer carries
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(refine_w ? a.w_offsets + nb0 * R : a.w_codes, refine_w && rows > 0 ? rows * R + 16 : 0);
  const __amdgpu_buffer_rsrc_t rxc = make_rsrc(a.x_codes, B * (K >> 1));
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(a.x_scales, B * (K >> 4));
  const __amdgpu_buffer_rsrc_t rxo = make_rsrc(refine_x ? a.x_offsets : a.x_codes, refine_x ? B * (K >> 2) : 0);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(refine_w ? a.w_mask : a.w_codes, refine_w ? K >> 5 : 0);
  const uint32_t crow = (uint32_t)(r * (K >> 1) + 32 * q);
  const uint32_t orow = (uint32_t)(r * R);

  unsigned char *wl = lds + (size_t)wave * (REF ? Lay::bytes6 : Lay::bytes4);
  unsigned char *wsc = wl;
  unsigned char *xsl = wl + Lay::xs;
  float *sxf = (float *)(wl + Lay::sx);
  unsigned char *dxl = wl + Lay::dx;
  uint4 *plan_sel = (uint4 *)(wl + Lay::plan);
  int32_t *plan_pos = (int32_t *)(plan_sel + 64);
  uint16_t *lut = (uint16_t *)(wl + Lay::lut);
  unsigned char *tsl = dxl;   // levels 2 and 4: the code transpose slot

  // 1. the range's scales and activation bytes, one 16-byte piece per lane
  //    per load: weight-scale piece j * 64 + l is row l % 16, chunk 4j + l / 16;
  //    activation pieces run token by token over the range
  constexpr int NX = Lay::tc * 8 / 64;   // activation-code loads per lane
  constexpr int NO = Lay::tc * 4 / 64;   // activation-offset loads per lane (level 6)
  uint32_t pw[kFp4Chunks / 4][4], px[NX][4], ps[4], pd[NO > 0 ? NO : 1][4], pm = 0;
  if (refine_w) {
    // mask bits of lane e = 4 * chunk + q: the 16 subgroups of its 64 elements
    const uint32_t o = (lane >> 2) < len ? (uint32_t)(8 * (c0 + (lane >> 2)) + 2 * (lane & 3)) : kOOB;
    pm = __builtin_amdgcn_raw_buffer_load_b16(rm, (int)o, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kFp4Chunks / 4; ++j) {
    const int p = 4 * j + q;
    const uint32_t o = p < len ? (uint32_t)(r * (K >> 4) + 16 * (c0 + p)) : kOOB;
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rsc, (int)o, 0, 0);
    pw[j][0] = v[0]; pw[j][1] = v[1]; pw[j][2] = v[2]; pw[j][3] = v[3];
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    const int p = 64 * j + lane;
    const int t = p / (8 * Lay::cap), w = p - t * 8 * Lay::cap;
    const uint32_t o = (t < B && w < 8 * len) ? (uint32_t)(t * (K >> 1) + 128 * c0 + 16 * w) : kOOB;
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rxc, (int)o, 0, 0);
    px[j][0] = v[0]; px[j][1] = v[1]; px[j][2] = v[2]; px[j][3] = v[3];
  }
  {
    const int t = lane / Lay::cap, c = lane - t * Lay::cap;
    const uint32_t o = (lane < Lay::tc && t < B && c < len) ? (uint32_t)(t * (K >> 4) + 16 * (c0 + c)) : kOOB;
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rxs, (int)o, 0, 0);
    ps[0] = v[0]; ps[1] = v[1]; ps[2] = v[2]; ps[3] = v[3];
  }
  if (REF) {
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int p = 64 * j + lane;
      const int t = p / (4 * Lay::cap), w = p - t * 4 * Lay::cap;
      const uint32_t o = (refine_x && t < B && w < 4 * len) ? (uint32_t)(t * (K >> 2) + 64 * c0 + 16 * w) : kOOB;
      const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rxo, (int)o, 0, 0);
      pd[j][0] = v[0]; pd[j][1] = v[1]; pd[j][2] = v[2]; pd[j][3] = v[3];
    }
  }
  vmem_fence();

  // 2. level 6: refined subgroups before the range, and the offset plan
  //    (the mask is shared by every row, so one plan serves the 16 rows)
  if (refine_w) {
    int32_t before = 0;
    const int64_t mdw = 2 * c0;   // mask dwords before the range
    for (int64_t i = lane; i < mdw; i += 64) before += __popc(ld_b32(rm, (uint32_t)(4 * i)));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
    const uint32_t m16 = pm & 0xFFFFu;
    const int32_t cnt = __popc(m16);
    int32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const PlanEntry pe = make_entry(m16, before + incl - cnt);
    plan_sel[lane] = make_uint4(pe.sel[0], pe.sel[1], pe.sel[2], pe.sel[3]);
    plan_pos[lane] = pe.pos;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t b = 4 * lane + 2 * j;
      *(uint32_t *)(lut + b) = offsets_to_e2m1(b | ((b + 1) << 8));
    }
  }

  // 3. the first PD chunks of weight codes (and level-6 offset windows).
  //    With ROWS, levels 2 and 4 load whole rows: load A brings rows 0..7 of
  //    the chunk (lane l: row l / 8), load B rows 8..15, each 8 lanes one
  //    128-byte row; lane slot s of row rho holds 16-byte piece s ^ (rho / 2)
  //    (the XOR keeps the transposed reads in process free of bank conflicts).
  //    Non-temporal: the codes are read once. Otherwise, and always at level 6
  //    (its offset windows follow it), the MFMA lane layout: lane (r, q)
  //    loads bytes 32q .. 32q + 31 of row r. Whole rows read faster (8 full
  //    128-byte lines per load instead of 16 half lines) but put an LDS round
  //    trip in each chunk: worth it when the launch has enough wavefronts to
  //    hide it.
  struct Buf {
    uint32_t c[8];   // 64 weight codes
    uint32_t o[3];   // offset dwords covering the lane's offset window
    uint32_t sh;     // byte position of the window in o
  };
  const uint32_t rowA = (uint32_t)(lane >> 3), rowB = rowA + 8;
  const uint32_t pA = (uint32_t)(((lane & 7) ^ (rowA >> 1)) * 16), pB = (uint32_t)(((lane & 7) ^ (rowB >> 1)) * 16);
  const uint32_t voA = P3 ? rowA * (uint32_t)(K >> 1) + pA : crow;
  const uint32_t voB = P3 ? rowB * (uint32_t)(K >> 1) + pB : crow + 16;
  auto load = [&](int i, Buf &b) {
    const bool live = i < len;
    const uint32_t so = live ? (uint32_t)((c0 + i) * 128) : 0u;
    const u32x4v lo = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(live ? voA : kOOB), (int)so, P3 ? 2 : 0);
    const u32x4v hi = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(live ? voB : kOOB), (int)so, P3 ? 2 : 0);
    b.c[0] = lo[0]; b.c[1] = lo[1]; b.c[2] = lo[2]; b.c[3] = lo[3];
    b.c[4] = hi[0]; b.c[5] = hi[1]; b.c[6] = hi[2]; b.c[7] = hi[3];
    if (refine_w) {
      const int32_t pos = live ? plan_pos[4 * i + q] : 0;
      const uint32_t at = orow + (uint32_t)pos;
      const u32x3v v = __builtin_amdgcn_raw_buffer_load_b96(ro, (int)(live ? at & ~3u : kOOB), 0, 0);
      b.o[0] = v[0]; b.o[1] = v[1]; b.o[2] = v[2];
      b.sh = at & 3u;
    }
  };
  Buf buf[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    load(u, buf[u]);
    vmem_fence();
  }

  // 4. prologue bytes to LDS (waits for them only: the code loads stay in flight)
#pragma unroll
  for (int j = 0; j < kFp4Chunks / 4; ++j)
    *(uint4 *)(wsc + r * kFp4Pitch + 16 * (4 * j + q)) = make_uint4(pw[j][0], pw[j][1], pw[j][2], pw[j][3]);
#pragma unroll
  for (int j = 0; j < NX; ++j)
    *(uint4 *)(xsl + 16 * (64 * j + lane)) = make_uint4(px[j][0], px[j][1], px[j][2], px[j][3]);
  if (lane < Lay::tc) {
    // a (token, chunk)'s 16 activation group scales as fp32
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ps[j], 1.0f, false);
      const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ps[j], 1.0f, true);
      *(float4v *)(sxf + 16 * lane + 4 * j) = float4v{v0[0], v0[1], v1[0], v1[1]};
    }
  }
  if (REF) {
    // 64 offsets (16 bytes) -> 64 E2M1 codes (32 bytes)
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      uint32_t e[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        e[2 * k] = offsets_to_e2m1(pd[j][k]);
        e[2 * k + 1] = offsets_to_e2m1(pd[j][k] >> 16);
      }
      *(uint4 *)(dxl + 32 * (64 * j + lane)) = make_uint4(e[0], e[1], e[2], e[3]);
      *(uint4 *)(dxl + 32 * (64 * j + lane) + 16) = make_uint4(e[4], e[5], e[6], e[7]);
    }
  }

  // A operand of MFMA m: lane (s = r, q) carries, in A row s, one group of
  // token ta(m, s) (levels 2/4: codes of token 2m + s / 8; level 6: codes of
  // token m for s < 8, its offsets d/2 for s >= 8) when (s & 7) / 2 == q:
  // group 4q + 2h + (s & 1) in the MFMA lane layout, 8h + (s & 7) with whole
  // rows. D row 4q + k of MFMA m belongs to token td(m, q) (2m + q / 2, or m).
  const bool a_slot = ((r & 7) >> 1) == q;
  const bool a_hi = (r & 1) != 0;
  const uint32_t a_off = P3 ? (uint32_t)(8 * (r & 7)) : (uint32_t)(32 * q + 8 * (r & 1));
  const uint32_t sxo = P3 ? (uint32_t)(4 * (q & 1)) : (uint32_t)(8 * (q & 1));
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;
  auto process = [&](int i, const Buf &b) {
    uint4 sel = make_uint4(0, 0, 0, 0);
    uint32_t wlo = 0, whi = 0;
    if (refine_w) {
      sel = plan_sel[4 * i + q];
      wlo = __builtin_amdgcn_alignbyte(b.o[1], b.o[0], b.sh);
      whi = __builtin_amdgcn_alignbyte(b.o[2], b.o[1], b.sh);
    }
    if (P3) {
      *(uint4 *)(tsl + 16 * lane) = make_uint4(b.c[0], b.c[1], b.c[2], b.c[3]);
      *(uint4 *)(tsl + 1024 + 16 * lane) = make_uint4(b.c[4], b.c[5], b.c[6], b.c[7]);
    }
    // weight group scales of the lane's D rows: 4 per half (whole rows) or
    // 8 per chunk (MFMA lane layout)
    float sw[8];
    {
      const uint2 sw2 = *(const uint2 *)(wsc + r * kFp4Pitch + 16 * i + (P3 ? 4 * (q & 1) : 8 * (q & 1)));
      const uint32_t sa = sw2.x, sb = P3 ? *(const uint32_t *)(wsc + r * kFp4Pitch + 16 * i + 8 + 4 * (q & 1)) : sw2.y;
      const auto w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sa, 1.0f, false);
      const auto w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sa, 1.0f, true);
      const auto w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false);
      const auto w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, true);
      sw[0] = w0[0]; sw[1] = w0[1]; sw[2] = w1[0]; sw[3] = w1[1];
      sw[4] = w2[0]; sw[5] = w2[1]; sw[6] = w3[0]; sw[7] = w3[1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x8v bw, bo;
      uint32_t wd[4];
      if (P3) {
        const uint4 wv = *(const uint4 *)(tsl + 128 * r + 16 * ((4 * h + q) ^ (r >> 1)));
        wd[0] = wv.x; wd[1] = wv.y; wd[2] = wv.z; wd[3] = wv.w;
      } else {
        wd[0] = b.c[4 * h]; wd[1] = b.c[4 * h + 1]; wd[2] = b.c[4 * h + 2]; wd[3] = b.c[4 * h + 3];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bw[k] = (int)(L == 2 ? autofp2_remap(wd[k]) : wd[k]);
        bw[4 + k] = 0;
      }
      if (refine_w) {
        // weight offsets d_W / 2 of the lane's 8 subgroup slots, as E2M1
        const uint32_t e0 = __builtin_amdgcn_perm(whi, wlo, h ? sel.z : sel.x);
        const uint32_t e1 = __builtin_amdgcn_perm(whi, wlo, h ? sel.w : sel.y);
        bo[0] = (int)(lut[e0 & 0xFFu] | ((uint32_t)lut[(e0 >> 8) & 0xFFu] << 16));
        bo[1] = (int)(lut[(e0 >> 16) & 0xFFu] | ((uint32_t)lut[e0 >> 24] << 16));
        bo[2] = (int)(lut[e1 & 0xFFu] | ((uint32_t)lut[(e1 >> 8) & 0xFFu] << 16));
        bo[3] = (int)(lut[(e1 >> 16) & 0xFFu] | ((uint32_t)lut[e1 >> 24] << 16));
        bo[4] = bo[5] = bo[6] = bo[7] = 0;
      }
      // the lane's 4 D rows <-> groups: whole rows 8h + 4 (q & 1) + k;
      // MFMA lane layout 8 (q & 1) + {0, 1, 4, 5}[k] + 2h
      const float s0 = P3 ? sw[4 * h + 0] : sw[0 + 2 * h], s1 = P3 ? sw[4 * h + 1] : sw[1 + 2 * h];
      const float s2 = P3 ? sw[4 * h + 2] : sw[4 + 2 * h], s3 = P3 ? sw[4 * h + 3] : sw[5 + 2 * h];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int ta = REF ? m : 2 * m + (r >> 3);
        const int td = REF ? m : 2 * m + (q >> 1);
        const unsigned char *ab = (REF && r >= 8 ? dxl : xsl) + ta * (Lay::cap * 128) + 128 * i + a_off +
                                  (P3 ? 64 * h : 16 * h);
        const uint2 xv = *(const uint2 *)ab;
        const bool live = a_slot && ta < B && (r < 8 || REF || BT > 1);
        const uint32_t xl = live ? xv.x : 0u, xh = live ? xv.y : 0u;
        i32x8v ax;
        ax[0] = (int)(a_hi ? 0u : xl);
        ax[1] = (int)(a_hi ? 0u : xh);
        ax[2] = (int)(a_hi ? xl : 0u);
        ax[3] = (int)(a_hi ? xh : 0u);
        ax[4] = ax[5] = ax[6] = ax[7] = 0;
        float4v d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            ax, bw, float4v{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, 127, 0, 127);
        if (refine_w) {
          // + A * (d_W / 2) at scale 2^-2 = A * d_W / 8
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ax, bo, d, 4, 4, 0, 127, 0, 125);
        }
        const float *sp = sxf + (td * Lay::cap + i) * 16;
        float x0, x1, x2, x3;
        if (P3) {
          const float4v v = *(const float4v *)(sp + 8 * h + sxo);
          x0 = v[0]; x1 = v[1]; x2 = v[2]; x3 = v[3];
        } else {
          const float4v va = *(const float4v *)(sp + sxo), vb = *(const float4v *)(sp + sxo + 4);
          x0 = h ? va[2] : va[0]; x1 = h ? va[3] : va[1]; x2 = h ? vb[2] : vb[0]; x3 = h ? vb[3] : vb[1];
        }
        float t = acc[m];
        t = fmaf(d[0], s0 * x0, t);
        t = fmaf(d[1], s1 * x1, t);
        t = fmaf(d[2], s2 * x2, t);
        t = fmaf(d[3], s3 * x3, t);
        acc[m] = t;
      }
    }
  };

  // 5. PD buffered chunks, each processed and then refilled PD chunks ahead
  for (int g = 0; g < len; g += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (g + u < len) process(g + u, buf[u]);
      vmem_fence();
      load(g + u + PD, buf[u]);
      vmem_fence();
    }
  }

  // 6. per MFMA: level 6 adds the offset rows (lane groups 2, 3) at a
  //    quarter into lane group 0; levels 2/4 add lane groups 0 + 1 (token
  //    2m) and 2 + 3 (token 2m + 1). Then the K-split wavefronts of each row
  //    tile are summed in LDS, [wave][token][row].
  float *red = (float *)lds;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = acc[m];
    if (REF) {
      v *= (q < 2 ? 1.0f : 0.25f);
      v += __shfl_xor(v, 32, 64);
    }
    v += __shfl_xor(v, 16, 64);
    const int td = REF ? m : 2 * m + (q >> 1);
    if ((REF ? q == 0 : (q & 1) == 0) && td < BT) red[(wave * BT + td) * 16 + r] = v;
  }
  __syncthreads();
  if (kw != 0 || rows == 0) return;
  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
  for (int e = lane; e < B * 16; e += 64) {
    const int t = e >> 4, rr = e & 15;
    if (rr >= rows) continue;
    float s = 0.f;
    for (int w = 0; w < WK; ++w) s += red[((wave + w) * BT + t) * 16 + rr];
    const float v = s * scale;
    if (a.y_dtype == AUTOFP_BF16) ((uint16_t *)a.y)[t * a.n + n0 + rr] = f32_to_bf16_rne(v);
    else ((float *)a.y)[t * a.n + n0 + rr] = v;
  }
}

// Chunks of code loads in flight: fewer as the token slots take registers.
// Level 6 runs up to 4 token slots (8 would spill: 16 MFMAs per half-chunk);
// the launcher sends 5-8 tokens at level 6 to the streaming kernel.
template <bool ROWS, int BT>
__global__ __launch_bounds__(1024) void gemv_fp4_kernel(LinearArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int D4 = BT <= 2 ? kFp4Depth : kFp4Depth / 2;
  constexpr int D6 = BT <= 2 ? kFp4Depth6 : kFp4Depth6 / 2;
  const int L = run_level(a);
  if (L == 6) {
    if constexpr (BT <= 4) fp4_tile<6, D6, false, BT>(a, lds);
  } else if (L == 2) {
    fp4_tile<2, D4, ROWS, BT>(a, lds);
  } else {
    fp4_tile<4, D4, ROWS, BT>(a, lds);
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

// XP: the activations are read packed (E2M1 codes, E4M3 scales and, at level
// 6, offset bytes: 0.5625 to 0.8125 B per element instead of the 2 B of the
// fp16 panel) and decoded in registers; K % 32 == 0. Every block reads all
// tokens' activations, so their bytes, not the weights', bound the launch.
template <int TT, int U, bool XP>
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
  const bool refine_x = XP && L == 6 && a.x_offsets != nullptr;

  float4v acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t cb = c0; cb < c1; cb += U) {
    uint4 cw[U];
    uint32_t sw[U];
    half8v xv[XP ? 1 : U][TT][4];
    uint4 xc[XP ? U : 1][TT];      // XP: 32 codes, their 2 scales and 8 offset bytes
    uint32_t xs[XP ? U : 1][TT];
    uint2 xo[XP ? U : 1][TT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      const int64_t ke = (c << 7) + (ks << 5);
      load_w(w, ke, c < c1, cw[u], sw[u]);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int64_t tok = 16 * t + r;
        if (XP) {
          const bool ok = (c < c1) && tok < a.b && ke < K;
          const int64_t tk = ok ? tok : 0, kk = ok ? ke : 0;
          xc[u][t] = ok ? *(const uint4 *)(a.x_codes + tk * (K >> 1) + (kk >> 1)) : make_uint4(0, 0, 0, 0);
          xs[u][t] = ok ? (uint32_t)*(const uint16_t *)(a.x_scales + tk * (K >> 4) + (kk >> 4)) : 0u;
          xo[u][t] = (ok && refine_x) ? *(const uint2 *)(a.x_offsets + tk * (K >> 2) + (kk >> 2)) : make_uint2(0, 0);
        } else {
          const bool tok_ok = (c < c1) && tok < a.b;
          const half8v *src = (const half8v *)(a.xh + (tok_ok ? tok : 0) * a.kpad + (c < c1 ? ke : 0));
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[u][t][i] = tok_ok ? src[i] : half8v{0, 0, 0, 0, 0, 0, 0, 0};
        }
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
        for (int i = 0; i < 4; ++i) {
          half8v xi;
          if (XP) {
            const uint32_t cwi = i == 0 ? xc[u][t].x : i == 1 ? xc[u][t].y : i == 2 ? xc[u][t].z : xc[u][t].w;
            const uint32_t obi = (i < 2 ? xo[u][t].x : xo[u][t].y) >> (16 * (i & 1));
            xi = __builtin_bit_cast(half8v, act_decode8_vals(cwi, xs[u][t] >> (8 * (i >> 1)), obi, refine_x));
          } else {
            xi = xv[u][t][i];
          }
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h[i], xi, acc[t], 0, 0, 0);
        }
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
  int waves;   // wavefronts per block = rt * wk
  int wk;      // wavefronts per row tile (K split)
  int rt;      // row tiles per block
  int pd;      // chunks in flight per wavefront (4 or 8)
  bool xlds;
  bool fast;
  size_t lds;
};

// The library's only host-side mutable state: a per-device cache of one
// device property (LDS bytes per block). Relaxed atomics make concurrent
// first calls benign: every writer stores the same value.
int max_lds_per_block() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
      v = 65536;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

StreamCfg stream_cfg(const LinearArgs &a) {
  StreamCfg c{};
  const int64_t nch = (a.k + kCh - 1) / kCh;
  const int64_t tiles = (a.n + 15) / 16;
  // wavefronts per tile (K split): about six wavefronts per CU, at least four
  // chunks per wavefront, and every wavefront's range within one offset plan
  int wk = 1;
  const int64_t want = 1536;
  while (wk < kMaxWaves && tiles * wk < want && nch / (2 * wk) >= 4) wk <<= 1;
  if (a.waves > 0) wk = a.waves;
  while (wk < kMaxWaves && (nch + wk - 1) / wk > kPlanChunks) wk <<= 1;
  // row tiles per block: share the LDS activation copy among up to 16 wavefronts
  int rt = 1;
  while (rt * wk * 2 <= 4 && tiles >= (int64_t)rt * 2 * 256) rt <<= 1;
  c.wk = wk;
  c.rt = rt;
  c.waves = wk * rt;
  // 4 chunks in flight per wavefront: 8 (at two wavefronts per SIMD, 256
  // VGPRs) measured slower on every decode shape
  c.pd = 4;
  c.fast = (a.k % kCh) == 0;
  const size_t lut = (size_t)kLutBytes;
  const size_t red = (size_t)c.waves * 64 * sizeof(float4v);
  const size_t msk = (size_t)mask_lds_bytes(a.k);
  const size_t xs = ((size_t)a.b * (size_t)(nch * kCh + 8) * sizeof(_Float16) + 128 + 15) & ~(size_t)15;
  const size_t plan = a.w_mask ? (size_t)c.waves * kPlanBytesPerWave : 0;
  const size_t with_x = msk + xs + plan, without_x = msk + plan;
  c.xlds = lut + (with_x > red ? with_x : red) <= (size_t)max_lds_per_block();
  c.lds = lut + (c.xlds ? (with_x > red ? with_x : red) : (without_x > red ? without_x : red));
  return c;
}

// Launch shape of the matrix-core GEMV for bt (1, 2, 4 or 8) token slots.
// Levels 2 and 4 (8 chunks in flight) take long K ranges and about 400 or
// more wavefronts: every wavefront's prologue costs the same few loads, so
// short ranges make the launch instruction-bound (measured at one token:
// Wqkv 6.4 us at one wavefront per tile, 7.7 at four; Wo 4.9 at two, 5.3 at
// four). A host-side level 2 with K up to 4096 (the digit remap adds to
// every chunk's arithmetic) takes about 1536 wavefronts, and two per tile on
// evenly split wide weights (one token, graphs of 9 launches: Wqkv 8.5 -> 7.4 us, Wo 6.1
// -> 5.9, Wgate|Wup 16.2 -> 15.8). Level 6 (or a device-side level) takes the streaming kernel's
// shape, about 1536 wavefronts. When the row tiles split evenly over the
// compute units, 256 blocks of tiles / 256 tiles each. Ranges are capped at
// the LDS staging capacity (16 chunks at one token, 32 / bt above).
struct Fp4Cfg {
  int wk, rt;
  size_t lds;
  bool ok;
};

int fp4_cap(int bt) { return bt == 1 ? kFp4Chunks : 32 / bt; }

size_t fp4_wave_lds(int bt, bool six) {
  switch (bt) {
    case 1: return six ? Fp4Lay<1>::bytes6 : Fp4Lay<1>::bytes4;
    case 2: return six ? Fp4Lay<2>::bytes6 : Fp4Lay<2>::bytes4;
    case 4: return six ? Fp4Lay<4>::bytes6 : Fp4Lay<4>::bytes4;
    default: return six ? Fp4Lay<8>::bytes6 : Fp4Lay<8>::bytes4;
  }
}

Fp4Cfg fp4_cfg(const LinearArgs &a, bool six, int bt) {
  Fp4Cfg c{};
  const int64_t nch = a.k / kCh;
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t kCUs = 256;
  const int64_t per_cu = tiles / kCUs;
  const int cap = fp4_cap(bt);
  const size_t wave_lds = fp4_wave_lds(bt, six);
  int wk = a.waves > 0 ? a.waves : 1;
  while ((nch + wk - 1) / wk > cap) ++wk;
  const bool two = !six && a.bits == 2 && a.bits_dev == nullptr;   // host-side level 2
  if (tiles % kCUs == 0 && per_cu >= 2 && per_cu * wk <= kMaxWaves &&
      (size_t)(per_cu * wk) * wave_lds <= (size_t)max_lds_per_block()) {
    c.rt = (int)per_cu;
    if (a.waves == 0 && (six || two)) {
      while (c.rt * wk * 2 <= kMaxWaves && nch / (2 * wk) >= 8 &&
             (size_t)(c.rt * wk * 2) * wave_lds <= (size_t)max_lds_per_block()) {
        wk *= 2;
        if (two) break;   // level 2: two wavefronts per tile
      }
    }
    c.wk = wk;
  } else if (!six && a.waves == 0) {
    while (tiles * wk < (two && nch <= kFp4Chunks ? 1536 : 384) && nch / (2 * wk) >= 4) wk <<= 1;
    c.wk = wk;
    c.rt = 1;
  } else {
    const StreamCfg sc = stream_cfg(a);
    c.wk = sc.wk > wk ? sc.wk : wk;
    while ((nch + c.wk - 1) / c.wk > cap) ++c.wk;
    c.rt = c.wk == sc.wk ? sc.rt : 1;
  }
  c.lds = (size_t)c.wk * c.rt * wave_lds;
  c.ok = c.wk * c.rt <= kMaxWaves && (nch + c.wk - 1) / c.wk <= cap && c.lds <= (size_t)max_lds_per_block();
  return c;
}

}  // namespace

int64_t xh_kpad(int64_t k) { return round_up(k, kCh); }

// 17-64 tokens with K % 64 == 0 on weights of 8192+ rows run the 64-token
// GEMM tile (enough row tiles to fill the chip); narrower weights the panel
// kernel. On the tile with four wavefront groups over K, 64 tokens took
// Wqkv 6144 x 4096 29.9 us (panel 44.2) but Wo 29.6 (26.1), Wdown
// 4096 x 14336 83.7 (72.1), and level 6 up to 1.6x the panel's time.
bool gemv_small_m_route(const LinearArgs &a) {
  return a.b > 16 && !gemv_batch_ok(a) && gemm_small_m_ok(a) && a.n >= 8192;
}

// 17+ tokens off the GEMM tile with K % 32 == 0 at a host-side level 2 or 4:
// the panel kernel reads the packed activations (no fp16 panel). 64 tokens:
// Wqkv 43.9 -> 29.5 us, Wo 26.0 -> 22.2, Wdown 71.1 -> 66.1 at level 4; at
// level 6 the offset decode made it slower (Wdown 101 -> 121 us), so level 6
// and a device-side level keep the fp16 panel.
bool gemv_panel_packed(const LinearArgs &a) {
  return a.b > 16 && !gemv_batch_ok(a) && !gemv_small_m_route(a) && (a.k & 31) == 0 && a.bits_dev == nullptr &&
         a.bits != 6;
}

// 9-16 tokens take the batched kernel on the larger weights (measured at 16
// tokens, graphs of 9 launches, levels 2/4/6: Wqkv 19.0/18.1/28.8 ->
// 14.9/13.6/20.5 us, Wgate|Wup 30.5/29.4/44.8 -> 27.2/23.1/40.6, Wdown
// 27.4/26.0/30.4 -> 19.6/17.1/30.8) and the streaming kernel on the smaller
// ones (Wo 10.4/10.1/16.1 against 12.1/11.3/17.6 us)
bool gemv_batch_route(const LinearArgs &a) {
  return a.b > 16 ? gemv_batch_ok(a) : (a.b > 8 && (a.n >= 6144 || a.k > 4096) && gemv_batch_ok(a));
}

bool gemv_needs_panel(const LinearArgs &a) {
  if (gemv_batch_route(a)) return false;
  if (a.b > 16) return !gemv_panel_packed(a);
  return !stream_cfg(a).xlds;
}

hipError_t launch_act_dequant(const LinearArgs &a, hipStream_t s) {
  const int64_t threads = a.b * (a.kpad / 8);
  hipLaunchKernelGGL(act_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const LinearArgs &a0, hipStream_t s) {
  // up to 8 tokens (4 at level 6) with K % 256 == 0: the fp4 matrix-core kernel
  const bool six0 = a0.bits_dev != nullptr || a0.bits == 6;
  if (a0.b <= (six0 ? 4 : 8) && a0.k % kCh == 0) {
    const bool six = six0;
    const int bt = a0.b == 1 ? 1 : a0.b == 2 ? 2 : a0.b <= 4 ? 4 : 8;
    const Fp4Cfg c = fp4_cfg(a0, six, bt);
    // on wide weights (1024+ row tiles) the short ranges of 8 token slots,
    // and level 6 at 4 (two chunks in flight), lose to the streaming kernel
    // (measured on Wgate|Wup: 22.6 vs 18.8 us at 8 tokens, level 4; 37.4 vs
    // 28.3 us at 4 tokens, level 6)
    const bool wide = (a0.n + 15) / 16 >= 1024;
    if (c.ok && !(wide && (bt == 8 || (bt == 4 && six)))) {
      LinearArgs a1 = a0;
      a1.wk = c.wk;
      const int64_t tiles = (a0.n + 15) / 16;
      const dim3 grid((unsigned)((tiles + c.rt - 1) / c.rt)), block((unsigned)(64 * c.wk * c.rt));
      // whole-row loads from 1024 wavefronts up (measured at one token:
      // Wgate|Wup, Wdown and the 70B shape 3-7 % faster; Wqkv and Wo,
      // 384-512 wavefronts, slower)
      const bool rows = (int64_t)grid.x * c.wk * c.rt >= 1024;
#define AFP_FP4(R, T) hipLaunchKernelGGL((gemv_fp4_kernel<R, T>), grid, block, c.lds, s, a1)
      if (bt == 1) { if (rows) AFP_FP4(true, 1); else AFP_FP4(false, 1); }
      else if (bt == 2) { if (rows) AFP_FP4(true, 2); else AFP_FP4(false, 2); }
      else if (bt == 4) { if (rows) AFP_FP4(true, 4); else AFP_FP4(false, 4); }
      else { if (rows) AFP_FP4(true, 8); else AFP_FP4(false, 8); }
#undef AFP_FP4
      return hipGetLastError();
    }
  }
  if (a0.b <= 16 && gemv_batch_route(a0)) return launch_gemv_batch(a0, s);
  if (a0.b <= 16) {
    const StreamCfg c = stream_cfg(a0);
    LinearArgs a1 = a0;
    a1.wk = c.wk;
    const int64_t tiles = (a0.n + 15) / 16;
    const dim3 grid((unsigned)((tiles + c.rt - 1) / c.rt)), block((unsigned)(64 * c.waves));
#define AFP_STREAM(X, F, P, R) hipLaunchKernelGGL((gemv_stream_kernel<X, F, P, R>), grid, block, c.lds, s, a1)
    // prologue items per thread: 4 covers one token; 16 the rest (4 would
    // leave larger batches on the loop, whose loads wait one by one)
    const int64_t items = a0.b * ((a0.k + kCh - 1) / kCh) * (kCh / 8);
    if (c.xlds && c.fast) {
      if (items <= 4 * 64 * (int64_t)c.waves) AFP_STREAM(true, true, 4, 4);
      else AFP_STREAM(true, true, 4, 16);
    } else if (c.xlds) {
      AFP_STREAM(true, false, 4, 4);
    } else {
      if (c.fast) AFP_STREAM(false, true, 4, 4); else AFP_STREAM(false, false, 4, 4);
    }
#undef AFP_STREAM
    return hipGetLastError();
  }
  // more than 16 tokens with K % 64 == 0: the batched kernel (slices of 64
  // tokens); otherwise, for wide weights, the 64-token GEMM tile, and slices
  // of at most 64 tokens on the panel kernel
  if (gemv_batch_ok(a0)) return launch_gemv_batch(a0, s);
  if (gemv_small_m_route(a0)) return launch_gemm_small_m(a0, s);
  for (int64_t t0 = 0; t0 < a0.b; t0 += 64) {
    LinearArgs a = a0;
    a.b = (a0.b - t0) < 64 ? (a0.b - t0) : 64;
    a.xh = a0.xh + t0 * a0.kpad;
    a.x_codes = a0.x_codes + t0 * (a0.k / 2);
    a.x_scales = a0.x_scales + t0 * (a0.k / 16);
    a.x_offsets = a0.x_offsets ? a0.x_offsets + t0 * (a0.k / 4) : nullptr;
    a.y = (char *)a0.y + t0 * a0.n * (a0.y_dtype == AUTOFP_BF16 ? 2 : 4);
    const dim3 grid((unsigned)((a.n + 15) / 16));
    const bool xp = gemv_panel_packed(a0);
#define AFP_PANEL(TT, U)                                                                      \
    if (xp) hipLaunchKernelGGL((gemv_panel_kernel<TT, U, true>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((gemv_panel_kernel<TT, U, false>), grid, dim3(256), 0, s, a)
    if (a.b <= 16) {
      AFP_PANEL(1, 4);
    } else if (a.b <= 32) {
      AFP_PANEL(2, 4);
    } else {
      AFP_PANEL(4, 2);
    }
#undef AFP_PANEL
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace afp
