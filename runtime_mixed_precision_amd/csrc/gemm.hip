// Prefill-phase AutoFP linear layer (GEMM) for gfx950.
//
// Same operation as the GEMV ("AutoEMatic", arXiv 2611.10165v1, §3.2, §4):
// Y = Xhat . What^T at level 2, 4 or 6, with exact products and fp32
// accumulation on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// The pages run this on FP4 tensor cores with E4M3 scales per 16 elements. The
// gfx950 scaled fp4/fp6/fp8 MFMA takes one power-of-two (E8M0) scale per 32
// elements and at most 4 significant bits per operand, which cannot hold
// B*(q + d/8) (up to 10 significant bits) exactly. The operands are therefore
// decoded into fp16 - exact - and multiplied at the fp16 MFMA rate.
//
// Three kernels:
//  - gemm_lds_kernel (K % 64 == 0, the prefill and batched-decode path): a
//    block of 8 or 16 wavefronts computes BM tokens x BN weight rows (256 x 256
//    or 256 x 128 for prefill, 64 x 64..256 for 17-64 decode tokens) in K steps
//    of 64 with two LDS stages; the fp16 activation panel goes memory -> LDS
//    with buffer_load ... lds, the packed weight tile is decoded in registers
//    and written to LDS (description above the kernel). The prefill tiles
//    (K <= 32768) let the two halves of the block load the weight steps in
//    turn, two steps ahead.
//  - gemm_kernel (any K % 16 == 0): 4 wavefronts on a 128 x 128 tile, both
//    operands through registers; the fallback for K % 64 != 0.
//  - gemv_fmt_kernel (the variant formats at 1-4 tokens): a vector GEMV over
//    the same weight decode, one wavefront per two weight rows.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "afp_act.h"
#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int BM = 128;   // tokens per tile
constexpr int BN = 128;   // weight rows per tile
constexpr int BK = 64;    // K per step
constexpr int LDSK = BK + 8;   // padded LDS row (halves)

__device__ __forceinline__ int run_level(const LinearArgs &a) {
  return a.bits_dev ? *a.bits_dev : a.bits;
}

struct TileRegs {
  uint4 cw;          // 32 weight codes
  uint32_t sw;       // two scale bytes
  uint32_t offs[8];  // offset bytes of the refined subgroups of this thread's 32 elements
  uint32_t mb;       // mask byte
  half8v xv[4];      // 32 activation halves
};

__global__ __launch_bounds__(256) void gemm_kernel(LinearArgs a) {
  __shared__ _Float16 Xs[BM][LDSK];
  __shared__ _Float16 Ws[BN][LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = a.k;
  const int64_t mt = blockIdx.x % ((a.b + BM - 1) / BM);
  const int64_t nt = blockIdx.x / ((a.b + BM - 1) / BM);
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int L = run_level(a);
  const bool refine_w = (L == 6) && a.w_mask != nullptr && a.w_offsets != nullptr;

  // loader mapping: thread -> (tile row, 32-element half)
  const int lr = tid >> 1;
  const int lh = tid & 1;
  const int64_t wrow = n0 + lr;
  const bool wrow_ok = wrow < a.n;
  const int64_t xrow = m0 + lr;
  const bool xrow_ok = xrow < a.b;
  const uint8_t *wcodes = a.w_codes + (wrow_ok ? wrow : 0) * (K >> 1);
  const uint8_t *wscl = a.w_scales + (wrow_ok ? wrow : 0) * (K >> 4);
  const uint8_t *woff = refine_w ? a.w_offsets + (wrow_ok ? wrow : 0) * (int64_t)a.n_refined : nullptr;
  const _Float16 *xsrc = a.xh + (xrow_ok ? xrow : 0) * a.kpad;
  const int64_t mbytes = (K + 31) >> 5;

  auto load_tile = [&](int64_t k0, TileRegs &t) {
    const int64_t ke = k0 + 32 * lh;
    t.cw = make_uint4(0, 0, 0, 0);
    t.sw = 0;
    t.mb = 0;
    if (wrow_ok && ke < K) {
      if ((K & 31) == 0) {
        t.cw = *(const uint4 *)(wcodes + (ke >> 1));
        t.sw = *(const uint16_t *)(wscl + (ke >> 4));
      } else {
        const uint2 lo = *(const uint2 *)(wcodes + (ke >> 1));
        t.cw.x = lo.x;
        t.cw.y = lo.y;
        t.sw = wscl[ke >> 4];
        if (ke + 16 < K) {
          const uint2 hi = *(const uint2 *)(wcodes + (ke >> 1) + 8);
          t.cw.z = hi.x;
          t.cw.w = hi.y;
          t.sw |= (uint32_t)wscl[(ke >> 4) + 1] << 8;
        }
      }
      if (refine_w) {
        const int64_t mi = ke >> 5;
        if (mi < mbytes) {
          t.mb = a.w_mask[mi];
          int32_t pos = a.prefix[mi];
          uint32_t m = t.mb;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            t.offs[s] = 0;
            if (((m >> s) & 1u) && pos < a.n_refined) t.offs[s] = woff[pos++];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.xv[i] = xrow_ok ? *(const half8v *)(xsrc + ke + 8 * i) : half8v{0, 0, 0, 0, 0, 0, 0, 0};
  };

  auto store_tile = [&](TileRegs &t) {
    uint32_t w4[4] = {t.cw.x, t.cw.y, t.cw.z, t.cw.w};
    if (L == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = autofp2_codes(w4[i]);
    }
    half8v h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = fp4x8_to_half8(w4[i]);
    if (refine_w && t.mb) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if ((t.mb >> s) & 1u) {
          half2v lo, hi;
          offsets_to_half4(t.offs[s], lo, hi);
          const half8v dl = (s & 1) ? half8v{0, 0, 0, 0, lo[0], lo[1], hi[0], hi[1]}
                                    : half8v{lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
          h[s >> 1] += dl;
        }
      }
    }
    const _Float16 b0 = (_Float16)e4m3_value(t.sw & 0xFFu);
    const _Float16 b1 = (_Float16)e4m3_value(t.sw >> 8);
    h[0] *= b0;
    h[1] *= b0;
    h[2] *= b1;
    h[3] *= b1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(half8v *)&Ws[lr][32 * lh + 8 * i] = h[i];
      *(half8v *)&Xs[lr][32 * lh + 8 * i] = t.xv[i];
    }
  };

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t nkt = (K + BK - 1) / BK;
  TileRegs cur;
  load_tile(0, cur);
  for (int64_t kt = 0; kt < nkt; ++kt) {
    store_tile(cur);
    __syncthreads();
    if (kt + 1 < nkt) load_tile((kt + 1) * BK, cur);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kof = kk * 16 + 8 * (lane >> 5);
      half8v af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const half8v *)&Xs[wm * 64 + i * 32 + (lane & 31)][kof];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *(const half8v *)&Ws[wn * 64 + j * 32 + (lane & 31)][kof];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
  // D[i][j]: lane holds column j = lane%32, rows 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= a.n) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= a.b) continue;
        const float val = acc[i][j][v] * scale;
        if (a.y_dtype == AUTOFP_BF16) ((uint16_t *)a.y)[m * a.n + n] = f32_to_bf16_rne(val);
        else ((float *)a.y)[m * a.n + n] = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-tile GEMM (K % 64 == 0): a block of NW wavefronts (8 or 16) computes
// BM tokens x BN weight rows in K steps of 64, with two LDS stages.
// Activation tiles (fp16 panel) go from memory straight to LDS with
// buffer_load ... lds (no registers, no ALU); weight tiles are loaded into
// registers, decoded to fp16 and written to LDS. The loads of step k + 1 are
// issued before the MFMAs of step k. LDS rows are 128 bytes (64 halves) with
// the 16-byte chunk index XOR-swizzled by (row / 2) % 8, so the fragment reads
// of a 32x32x16 MFMA (32 rows, one chunk) spread over all banks. The
// wavefronts form a WGM x (NW / WGM) grid over the tile, each running a grid
// of v_mfma_f32_32x32x16_f16 tiles over its part.
// ---------------------------------------------------------------------------

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
typedef uint32_t u32x6v __attribute__((ext_vector_type(6)));
typedef _Float16 half32v __attribute__((ext_vector_type(32)));
#define AFP_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kBM2 = 256;
constexpr int kGemmWaves = 16;  // wavefronts per prefill block (four per SIMD, 128 VGPRs each)
constexpr int kDecodeWaves = 8; // wavefronts per 64-token block
constexpr int kBK2 = 64;
constexpr size_t kTabBytes = 2 * 256 * 8;   // level-6 decode tables of gemm_lds_kernel
constexpr int64_t kAltMaxK = 32768;         // K bound of the alternating-group prefill tiles (mask in LDS)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

// LDS byte offset of 16-byte chunk c (0..7) of tile row r: the chunk index is
// XORed with (r / 2) % 8, so the 16 rows at one chunk that a b128 LDS access
// serves per cycle fall on 16 distinct 16-byte bank groups (64 banks)
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) { return r * 128u + ((c ^ ((r >> 1) & 7u)) << 4); }

// One weight item, 32 elements of one row, to fp16: c (16 bytes of E2M1
// codes; FP6G: c and cx, 24 bytes of E2M3 codes), s2 (the two E4M3 scale
// bytes of its 16-element groups, low byte first) and, when refine, the offset
// window of its refined subgroups (AUTOFP6 / AUTOFP6E: o, 12 bytes; AUTOFP8:
// o4 and o5, 20 bytes) whose first offset starts sh bytes in, with m the
// item's mask byte. h[p] = elements 8p .. 8p + 7, times their group scale.
// Tables: dtab / stab (AUTOFP6, AUTOFP6E) or t8 (AUTOFP8), as filled by the
// kernels below. PK6: FP6G codes through the 32-element fp6 conversion.
template <int FMT, bool PK6 = false>
__device__ __forceinline__ void decode_w32(const u32x4v c, const u32x2v cx, uint32_t s2, const u32x3v o,
                                           const u32x4v o4, uint32_t o5, uint32_t m, uint32_t sh, int L,
                                           bool refine, const uint2 *dtab, const uint2 *stab, const uint32_t *t8,
                                           half8v h[4]) {
  constexpr bool F8 = FMT == AUTOFP_FMT_AUTOFP8;
  constexpr bool G6 = FMT == AUTOFP_FMT_FP6G;
  if constexpr (G6 && PK6) {
    // 32 six-bit E2M3 codes in 24 bytes (code i at bits [6i+5:6i] of the
    // six little-endian dwords) to fp16 in one conversion (exact; scale 1)
    const u32x6v src = {c[0], c[1], c[2], c[3], cx[0], cx[1]};
    const half32v v = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(src, 1.0f);
    h[0] = __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7);
    h[1] = __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15);
    h[2] = __builtin_shufflevector(v, v, 16, 17, 18, 19, 20, 21, 22, 23);
    h[3] = __builtin_shufflevector(v, v, 24, 25, 26, 27, 28, 29, 30, 31);
  } else if constexpr (G6) {
    // the same bits field by field: 8 codes (48 bits) per fragment, at bits
    // 0, 48, 96 and 144 of the six dwords (no 32-register result, for the
    // GEMM tiles whose register budget it would exceed)
    const uint64_t win4[4] = {((uint64_t)c[1] << 32) | c[0], (((uint64_t)c[2] << 32) | c[1]) >> 16,
                              ((uint64_t)cx[0] << 32) | c[3], (((uint64_t)cx[1] << 32) | cx[0]) >> 16};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t win = win4[j];
      half2v p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p[e] = e2m3x2_to_half2((uint32_t)(win >> (12 * e)) & 63u, (uint32_t)(win >> (12 * e + 6)) & 63u);
      h[j] = half8v{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
    }
  } else {
    uint32_t w4[4] = {c[0], c[1], c[2], c[3]};
    if (L == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w4[j] = autofp2_codes(w4[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = fp4x8_to_half8(w4[j]);
  }
  if (F8 && refine) {
    // the (at most 8) two-byte offset words of these 32 elements, in
    // subgroup order, from the 20 loaded bytes shifted by the misalignment
    const uint32_t W0 = __builtin_amdgcn_alignbyte(o4[1], o4[0], sh);
    const uint32_t W1 = __builtin_amdgcn_alignbyte(o4[2], o4[1], sh);
    const uint32_t W2 = __builtin_amdgcn_alignbyte(o4[3], o4[2], sh);
    const uint32_t W3 = __builtin_amdgcn_alignbyte(o5, o4[3], sh);
    const uint64_t lo = (uint64_t)W0 | ((uint64_t)W1 << 32), hi = (uint64_t)W2 | ((uint64_t)W3 << 32);
    uint32_t wd[8];
    uint32_t j = 0;
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) {
      const uint32_t on = (m >> sg) & 1u;
      const uint64_t src = j < 4 ? lo : hi;
      wd[sg] = on ? (uint32_t)(src >> (16 * (j & 3))) & 0xFFFFu : 0u;
      j += on;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a0 = wd[2 * p], a1 = wd[2 * p + 1];
      h[p] += __builtin_bit_cast(half8v, make_uint4(t8[a0 & 0xFFu], t8[a0 >> 8], t8[a1 & 0xFFu], t8[a1 >> 8]));
    }
  } else if (!G6 && refine) {
    // the (at most 8) offset bytes of these 32 elements, in subgroup order;
    // one byte per subgroup (0 where not refined) via a byte permute
    const uint32_t lo = __builtin_amdgcn_alignbyte(o[1], o[0], sh);
    const uint32_t hi = __builtin_amdgcn_alignbyte(o[2], o[1], sh);
    const uint2 sel = stab[m & 0xFFu];
    const uint32_t E[2] = {__builtin_amdgcn_perm(hi, lo, sel.x), __builtin_amdgcn_perm(hi, lo, sel.y)};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint2 de = dtab[(E[p >> 1] >> (16 * (p & 1))) & 0xFFu];
      const uint2 dd = dtab[(E[p >> 1] >> (16 * (p & 1) + 8)) & 0xFFu];
      const half8v dl = __builtin_bit_cast(half8v, make_uint4(de.x, de.y, dd.x, dd.y));
      if constexpr (FMT == AUTOFP_FMT_AUTOFP6E) {
        // delta = d/8 * 2^e of each element's E2M1 value
        const uint4 hv = __builtin_bit_cast(uint4, h[p]);
        const uint4 fv = make_uint4(__builtin_bit_cast(uint32_t, pow2e_h2(__builtin_bit_cast(half2v, hv.x))),
                                    __builtin_bit_cast(uint32_t, pow2e_h2(__builtin_bit_cast(half2v, hv.y))),
                                    __builtin_bit_cast(uint32_t, pow2e_h2(__builtin_bit_cast(half2v, hv.z))),
                                    __builtin_bit_cast(uint32_t, pow2e_h2(__builtin_bit_cast(half2v, hv.w))));
        h[p] += dl * __builtin_bit_cast(half8v, fv);
      } else {
        h[p] += dl;
      }
    }
  }
  const _Float16 b0 = (_Float16)e4m3_value(s2 & 0xFFu);
  const _Float16 b1 = (_Float16)e4m3_value((s2 >> 8) & 0xFFu);
  h[0] *= b0;
  h[1] *= b0;
  h[2] *= b1;
  h[3] *= b1;
}

// Level-6 decode tables in LDS (block-wide fill; the caller synchronizes):
// AUTOFP8: t8[byte] = the two fp16 offsets d/8 of a byte of two 4-bit
// offsets; otherwise dtab[byte] = the four fp16 offsets d/8 of an offset byte
// and stab[mask byte] = the byte selectors that spread a row's compacted
// offset bytes over the 8 subgroups of 32 elements (0x0C: no offset).
template <int FMT>
__device__ __forceinline__ void fill_decode_tables(uint2 *dtab, uint2 *stab, int L) {
  if constexpr (FMT == AUTOFP_FMT_AUTOFP8) {
    uint32_t *t8 = (uint32_t *)dtab;
    for (int i = (int)threadIdx.x; i < 256; i += (int)blockDim.x)
      t8[i] = __builtin_bit_cast(uint32_t, half2v{delta8_h((uint32_t)i, L == 6), delta8_h((uint32_t)i >> 4, L == 6)});
  } else {
    for (int i = (int)threadIdx.x; i < 256; i += (int)blockDim.x) {
      dtab[i] = delta_words((uint32_t)i);
      uint32_t sel[2] = {0, 0}, j = 0;
      for (int sg = 0; sg < 8; ++sg) {
        const uint32_t on = ((uint32_t)i >> sg) & 1u;
        sel[sg >> 2] |= (on ? j : 0x0Cu) << (8 * (sg & 3));
        j += on;
      }
      stab[i] = make_uint2(sel[0], sel[1]);
    }
  }
}

// NW wavefronts (8 or 16: two or four per SIMD, so one wavefront's decode
// and waits overlap the others' MFMAs) in a WGM x NW/WGM grid over the
// BM x BN tile (WGM = 4 for 16 wavefronts on 256 tokens, else 2).
//
// KG > 1 (batched decode): KG groups of NW wavefronts share the block's tile,
// each group running the K loop over its own quarter (half, ...) of K with its
// own two LDS stages, so KG times as many loads are in flight per tile while
// every weight and activation byte is still read once; a step past a group's
// range (or past K) loads zeros. At the end the groups' accumulators are
// summed through LDS in group order (deterministic) by group 0.
//
// ALT (prefill tiles, K <= kAltMaxK): the weight steps alternate between the
// two halves of the wavefronts (the schedule is described at the loop).
//
// FMT (autofp_format) selects the weight decode: AUTOFP6 (the default) and
// AUTOFP6E (its offsets scaled by 2^e of each element's E2M1 value) read one
// offset byte per refined subgroup; AUTOFP8 two (4-bit d, clamped to
// [-2, +1] at level 6); FP6G reads 24 bytes of E2M3 codes per 32 elements and
// no offsets.
template <int BM, int BN, int NW, int KG = 1, int FMT = AUTOFP_FMT_AUTOFP6, bool ALT = false>
__global__ __launch_bounds__(64 * NW * KG) void gemm_lds_kernel(LinearArgs a) {
  constexpr int WGM = (NW >= 16 && BM >= 256) ? 4 : 2;   // wavefronts along M
  constexpr int WGN = NW / WGM;                         // wavefronts along N
  constexpr int WM = BM / WGM;        // tokens per wavefront
  constexpr int WN = BN / WGN;        // weight rows per wavefront
  constexpr int TJ = WN / 32;         // 32-row MFMA tiles per wavefront along N
  constexpr int TI = WM / 32;         // 32-token MFMA tiles per wavefront along M
  constexpr int A_BYTES = BM * kBK2 * 2;
  constexpr int W_BYTES = BN * kBK2 * 2;
  constexpr int STAGE = A_BYTES + W_BYTES;
  constexpr int WITEMS = 2 * BN;              // (row, 32-element half) weight items per step
  constexpr int HPT = WITEMS >= 128 * NW ? 2 : 1;   // items per thread (threads past WITEMS idle)
  constexpr int APW = BM / 8 / NW;            // activation copy instructions per wavefront and step
  static_assert(APW >= 1, "at least one activation copy per wavefront");
  static_assert(WITEMS == 64 * NW * HPT || (HPT == 1 && WITEMS < 64 * NW), "weight items per thread");
  static_assert(!ALT || (KG == 1 && WITEMS <= 32 * NW), "alternating weight groups: one item per thread of a half");
  extern __shared__ __align__(16) unsigned char lds[];

  const int kg = KG > 1 ? (int)(threadIdx.x / (64 * NW)) : 0;   // K group
  const int tid = KG > 1 ? (int)(threadIdx.x % (64 * NW)) : (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t K = a.k;
  unsigned char *glds = lds + kg * 2 * STAGE;   // this group's two stages
  const int64_t mtiles = (a.b + BM - 1) / BM;
  const int64_t mt = blockIdx.x % mtiles;
  const int64_t nt = blockIdx.x / mtiles;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  constexpr bool F8 = FMT == AUTOFP_FMT_AUTOFP8;
  constexpr bool G6 = FMT == AUTOFP_FMT_FP6G;
  constexpr int64_t OW = F8 ? 2 : 1;                    // offset bytes per refined subgroup
  const int L = run_level(a);
  const bool refine_w = !G6 && (L == 6 || (F8 && L == 8)) && a.w_mask != nullptr && a.w_offsets != nullptr &&
                        a.n_refined > 0;
  const int64_t R = a.n_refined;
  const int64_t CB = G6 ? 3 * K / 4 : K / 2;            // code bytes per weight row

  // level 6: per-block tables after the stages. dtab[byte] = the four fp16
  // offsets d/8 of an offset byte; stab[mask byte] = the byte selectors that
  // spread a row's compacted offset bytes over the 8 subgroups of 32
  // elements (0x0C: no offset). A lookup replaces a few dozen bit operations
  // per 32 decoded weights. AUTOFP8: t8[byte] = the two fp16 offsets d/8 of
  // a byte of two 4-bit offsets.
  // (ALT: in an array of their own, which no copy into the stages can touch,
  // so reading them waits for no copy in flight)
  __shared__ uint2 tabs_alt[ALT ? 512 : 1];
  uint2 *dtab = ALT ? tabs_alt : (uint2 *)(lds + KG * 2 * STAGE);
  uint2 *stab = dtab + 256;
  uint32_t *t8 = (uint32_t *)dtab;
  // ALT: the weight mask and its prefix table in LDS (K <= kAltMaxK), so a
  // step's offset loads depend on no other load
  __shared__ uint8_t mask_l[ALT ? kAltMaxK / 32 : 1];
  __shared__ int32_t pref_l[ALT ? kAltMaxK / 32 + 1 : 1];
  if (refine_w) {
    fill_decode_tables<FMT>(dtab, stab, L);
    if constexpr (ALT) {
      for (int64_t i = threadIdx.x; i < K / 32; i += blockDim.x) mask_l[i] = a.w_mask[i];
      for (int64_t i = threadIdx.x; i <= K / 32; i += blockDim.x) pref_l[i] = a.prefix[i];
    }
    __syncthreads();
  }

  // activation panel [b][kpad] fp16, this block's BM rows only (so a panel
  // of any size is addressed with 32-bit offsets: BM * kpad * 2 < 2^31 for
  // k <= 2^22, which the entry points check); rows past b read as zero
  const int64_t mrows = (a.b - m0) < BM ? (a.b - m0) : BM;
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.xh + m0 * a.kpad, mrows * a.kpad * 2);
  // weight rows of this block: rows past n read as zero
  const int64_t nrows = (a.n - n0) < BN ? (a.n - n0) : BN;
  const __amdgpu_buffer_rsrc_t rc = rsrc(a.w_codes + n0 * CB, nrows * CB);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.w_scales + n0 * (K >> 4), nrows * (K >> 4));
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(refine_w ? a.w_offsets + n0 * R * OW : a.w_codes, refine_w ? nrows * R * OW + 16 : 0);

  // DMA mapping: instruction d of a wavefront covers A rows 8 (APW wave + d) ..
  // + 7; lane i -> row + i / 8, LDS chunk i % 8 (global chunk (i % 8) ^ ((row / 2) % 8))
  const uint32_t arow_l = (uint32_t)(lane >> 3);
  auto issue_a = [&](int64_t k0, int stage) {
    unsigned char *base = glds + stage * STAGE;
#pragma unroll
    for (int d = 0; d < APW; ++d) {
      const uint32_t r = (uint32_t)(8 * (APW * wave + d)) + arow_l;   // tile row 0..255
      const uint32_t cg = (uint32_t)(lane & 7) ^ ((r >> 1) & 7u);
      const uint32_t off = ((int64_t)r < mrows && k0 < K) ? (uint32_t)(((int64_t)r * a.kpad + k0 + 8 * cg) * 2) : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, AFP_LDS(base + 8 * (APW * wave + d) * 128), 16, (int)off, 0, 0, 0);
    }
  };

  // weight rows of this thread: halves h0 .. h0 + HPT - 1 of row wr
  // ALT: the two halves of the block's wavefronts (wg = 0, 1) take the
  // weight steps in turn, each thread of a half one item
  const int wg = ALT ? wave / (NW / 2) : 0;
  const int tw = ALT ? tid % (32 * NW) : tid;
  const int wr = (HPT == 2) ? tw : (tw >> 1);
  const int h0 = (HPT == 2) ? 0 : (tw & 1);
  const bool w_thread = tw < WITEMS / HPT;   // whole wavefronts: WITEMS is a multiple of 64
  struct WRegs {
    u32x4v c[HPT];
    u32x2v cx[HPT];   // FP6G: the last 8 of the 24 code bytes
    uint32_t s;
    u32x3v o[HPT];
    u32x4v o4[HPT];   // AUTOFP8: 20 bytes of compacted offsets
    uint32_t o5[HPT];
    int32_t pos[HPT];
    uint32_t mb[HPT];
  };
  // a step past K (a K group's tail) loads zeros: out-of-range buffer offsets,
  // and no refined subgroups
  auto load_w = [&](int64_t k0, WRegs &w) {
    const bool kin = k0 < K;
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int64_t ke = k0 + 32 * (h0 + i);
      if constexpr (G6) {
        const int off = (int)(wr * CB + 3 * ke / 4);
        w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, kin ? off : (int)0x80000000u, 0, 0);
        w.cx[i] = __builtin_amdgcn_raw_buffer_load_b64(rc, kin ? off + 16 : (int)0x80000000u, 0, 0);
      } else {
        w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, kin ? (int)(wr * (K >> 1) + (ke >> 1)) : (int)0x80000000u,
                                                       0, 0);
      }
    }
    if (HPT == 2 || ALT) {
      // ALT: the dword of the step's four scale bytes (both halves), so no
      // sub-dword result is widened after the load
      w.s = __builtin_amdgcn_raw_buffer_load_b32(rs, kin ? (int)(wr * (K >> 4) + (k0 >> 4)) : (int)0x80000000u, 0, 0);
    } else {
      w.s = __builtin_amdgcn_raw_buffer_load_b16(
          rs, kin ? (int)(wr * (K >> 4) + ((k0 + 32 * h0) >> 4)) : (int)0x80000000u, 0, 0);
    }
    if (refine_w) {
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int64_t mi = kin ? (k0 >> 5) + h0 + i : 0;   // mask byte (32 elements)
        if constexpr (ALT) {
          // mask byte and prefix are read again from LDS at the decode, so
          // they are not held in registers between the two steps
          w.pos[i] = pref_l[mi];
        } else {
          w.mb[i] = kin ? a.w_mask[mi] : 0u;
          w.pos[i] = a.prefix[mi];
        }
        if constexpr (F8) {
          const uint32_t al = (uint32_t)(((wr * R + w.pos[i]) * 2) & ~(int64_t)3);
          w.o4[i] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)al, 0, 0);
          w.o5[i] = __builtin_amdgcn_raw_buffer_load_b32(ro, (int)(al + 16), 0, 0);
        } else {
          const uint32_t al = (uint32_t)((wr * R + w.pos[i]) & ~(int64_t)3);
          w.o[i] = __builtin_amdgcn_raw_buffer_load_b96(ro, (int)al, 0, 0);
        }
      }
    }
  };
  // k0: the step's first element (read by ALT, which takes the item's mask
  // byte and prefix from LDS here)
  auto store_w = [&](const WRegs &w, int stage, int64_t k0) {
    unsigned char *base = glds + stage * STAGE + A_BYTES;
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      half8v h[4];
      const uint32_t sbytes = (HPT == 2) ? (w.s >> (16 * i)) : ALT ? (w.s >> (16 * h0)) : w.s;
      uint32_t mb = 0, sh = 0;
      if (refine_w) {
        if constexpr (ALT) {
          const int64_t mi = (k0 >> 5) + h0 + i;
          mb = mask_l[mi];
          sh = (uint32_t)(((wr * R + pref_l[mi]) * OW) & 3);
        } else {
          mb = w.mb[i];
          sh = (uint32_t)(((wr * R + w.pos[i]) * OW) & 3);
        }
      }
      decode_w32<FMT>(w.c[i], w.cx[i], sbytes, w.o[i], w.o4[i], w.o5[i], mb, sh, L, refine_w, dtab, stab, t8, h);
#pragma unroll
      for (int j = 0; j < 4; ++j) *(half8v *)(base + swz((uint32_t)wr, (uint32_t)(4 * (h0 + i) + j))) = h[j];
    }
  };

  float16v acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // K steps of this group: [kb, kb + nkt) (the same count in every group)
  const int64_t nkt = (K / kBK2 + KG - 1) / KG;
  const int64_t kb = nkt * kg;
  WRegs wreg;
  if constexpr (ALT) {
    // Weight step s is loaded by half s % 2 at the top of step s - 2 and
    // decoded into its LDS stage at the end of step s - 1: two steps for the
    // loads, one register set per thread. At the end of a step the half
    // that loaded waits for all but its own new loads (issued after the
    // activation copy, and the counter retires loads in issue order), the
    // other half for everything; then one barrier.
    constexpr int NWL = (G6 ? 2 : 1) + 1;            // weight loads per step: codes, scales
    constexpr int NWR = NWL + (F8 ? 2 : 1);          // and the offset window
    static_assert(NWR <= 15, "vmcnt field");
    auto wait_step = [&](bool keep_w) {
      if (!keep_w) __builtin_amdgcn_s_waitcnt((7 << 4));                 // vmcnt(0) lgkmcnt(0)
      else if (refine_w) __builtin_amdgcn_s_waitcnt(NWR | (7 << 4));     // vmcnt(NWR) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(NWL | (7 << 4));                   // vmcnt(NWL) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    issue_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (w_thread) load_w((int64_t)wg * kBK2, wreg);
    __builtin_amdgcn_sched_barrier(0);
    if (wg == 0 && w_thread) store_w(wreg, 0, 0);
    wait_step(wg == 1 && w_thread);
    // one step; LOAD / STORE: this half's role in it (compile-time, so the
    // compiler's own wait counts see which loads are in flight)
    auto step = [&](int64_t kt, auto load_role, auto store_role) {
      constexpr bool LOAD = decltype(load_role)::value, STORE = decltype(store_role)::value;
      // the stage index stays a run-time value, so the unrolled steps share one
      // set of LDS fragment addresses instead of holding one per stage
      int st = (int)(kt & 1);
      asm volatile("" : "+s"(st));
      const bool more = kt + 1 < nkt;
      if (more) issue_a((kt + 1) * kBK2, st ^ 1);
      __builtin_amdgcn_sched_barrier(0);   // the weight loads after the copy (the wait count relies on it)
      if (LOAD && w_thread) load_w((kt + 2) * kBK2, wreg);
      __builtin_amdgcn_sched_barrier(0);
      const unsigned char *As = glds + st * STAGE;
      const unsigned char *Wsb = As + A_BYTES;
#pragma unroll
      for (int kk = 0; kk < kBK2 / 16; ++kk) {
        const uint32_t ch = (uint32_t)(2 * kk + (lane >> 5));
        half8v af[TI], bf[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i)
          af[i] = *(const half8v *)(As + swz((uint32_t)(wm * WM + 32 * i + (lane & 31)), ch));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bf[j] = *(const half8v *)(Wsb + swz((uint32_t)(wn * WN + 32 * j + (lane & 31)), ch));
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if (STORE && more && w_thread) store_w(wreg, st ^ 1, (kt + 1) * kBK2);
      wait_step(LOAD && w_thread);
    };
    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    // half 0 loads on even steps and stores on odd ones, half 1 the reverse
    int64_t kt = 0;
    if (wg == 0) {
      for (; kt + 1 < nkt; kt += 2) {
        step(kt, T_{}, F_{});
        step(kt + 1, F_{}, T_{});
      }
      if (kt < nkt) step(kt, T_{}, F_{});
    } else {
      for (; kt + 1 < nkt; kt += 2) {
        step(kt, F_{}, T_{});
        step(kt + 1, T_{}, F_{});
      }
      if (kt < nkt) step(kt, F_{}, T_{});
    }
    __builtin_amdgcn_s_waitcnt(0);   // the loads past K (which return zeros) have retired
  } else {
  issue_a(kb * kBK2, 0);
  if (w_thread) {
    load_w(kb * kBK2, wreg);
    store_w(wreg, 0, kb * kBK2);
  }
  __builtin_amdgcn_s_waitcnt(0);   // every load of step 0 (the activation copy included) has landed
  __syncthreads();
  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int st = (int)(kt & 1);
    const bool more = kt + 1 < nkt;
    if (more) {
      issue_a((kb + kt + 1) * kBK2, st ^ 1);
      if (w_thread) load_w((kb + kt + 1) * kBK2, wreg);
    }
    const unsigned char *As = glds + st * STAGE;
    const unsigned char *Wsb = As + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < kBK2 / 16; ++kk) {
      const uint32_t ch = (uint32_t)(2 * kk + (lane >> 5));
      half8v af[TI], bf[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        af[i] = *(const half8v *)(As + swz((uint32_t)(wm * WM + 32 * i + (lane & 31)), ch));
#pragma unroll
      for (int j = 0; j < TJ; ++j) bf[j] = *(const half8v *)(Wsb + swz((uint32_t)(wn * WN + 32 * j + (lane & 31)), ch));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more && w_thread) store_w(wreg, st ^ 1, (kb + kt + 1) * kBK2);
    __builtin_amdgcn_s_waitcnt(0);   // the next step's activation copy has landed
    __syncthreads();
  }
  }

  if (KG > 1) {
    // groups 1 .. KG-1 leave their accumulators in LDS (lane-minor), group 0
    // adds them in group order
    float *red = (float *)lds;
    constexpr int PER = TI * TJ * 16;   // accumulator floats per lane
    if (kg > 0) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            red[(((kg - 1) * NW + wave) * PER + (i * TJ + j) * 16 + v) * 64 + lane] = acc[i][j][v];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[i][j][v] += red[(((g - 1) * NW + wave) * PER + (i * TJ + j) * 16 + v) * 64 + lane];
  }

  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
  // D tile (i, j): lane holds weight row 32 j + lane % 32 and tokens
  // 8 (v / 4) + 4 (lane / 32) + v % 4 of the 32-token tile i
  const bool out_bf16 = a.y_dtype == AUTOFP_BF16;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t n = n0 + wn * WN + 32 * j + (lane & 31);
    if (n >= a.n) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t mb0 = m0 + wm * WM + 32 * i + 4 * (lane >> 5);
      const bool full = m0 + wm * WM + 32 * i + 32 <= a.b;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mb0 + 8 * (v >> 2) + (v & 3);
        if (!full && m >= a.b) continue;
        const float val = acc[i][j][v] * scale;
        if (out_bf16) ((uint16_t *)a.y)[m * a.n + n] = f32_to_bf16_rne(val);
        else ((float *)a.y)[m * a.n + n] = val;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Variant formats at 1-4 tokens: vector GEMV
// ---------------------------------------------------------------------------
//
// A variant weight element B (q + delta) or an E2M3 code needs more than the
// four significant bits the fp4 matrix cores take, and a 64-token GEMM tile
// at one token leaves most of the chip idle ([AE] App. I Table 10, App. B.2:
// the formats; the product is the one the GEMM tiles compute). Here a
// wavefront owns RPW weight rows and its lanes split K into 32-element items:
// lane l takes items l, l + 64, ... of each row, decodes them with decode_w32
// (the GEMM tiles' own weight decode: fp16, exact, group scales applied) and
// accumulates their dot products with the fp16 activations in fp32
// (v_dot2_f32_f16, products exact in fp32); the lanes' sums are added across
// the wavefront at the end in one fixed order. The activations come from LDS,
// decoded there by the block (1-2 tokens), or from the fp16 panel of the
// workspace. TB >= b tokens (absent tokens read as zero).
// The time is mostly the decode's vector ALU (a wave64 instruction per four
// cycles on each SIMD), so FP6G takes its codes through the 32-element fp6
// conversion.

// Sum of the wavefront's values, the same in every lane, through DPP row
// moves and the row swaps (quad pairs, quads, half rows, rows, row pairs,
// halves: one fixed order).
__device__ __forceinline__ float wave_sum_f(float v) {
  auto dadd = [](float x, int ctrl) -> float {
    int y = 0;
    switch (ctrl) {   // the DPP control must be a constant
      case 0: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false); break;   // quad xor 1
      case 1: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false); break;   // quad xor 2
      case 2: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false); break;  // row half mirror
      default: y = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false); break; // row mirror
    }
    return x + __int_as_float(y);
  };
  v = dadd(v, 0);
  v = dadd(v, 1);
  v = dadd(v, 2);
  v = dadd(v, 3);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float dot8(half8v w, half8v x, float acc) {
  acc = __builtin_amdgcn_fdot2(half2v{w[0], w[1]}, half2v{x[0], x[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2v{w[2], w[3]}, half2v{x[2], x[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2v{w[4], w[5]}, half2v{x[4], x[5]}, acc, false);
  return __builtin_amdgcn_fdot2(half2v{w[6], w[7]}, half2v{x[6], x[7]}, acc, false);
}

constexpr int kFmtGemvWaves = 4;    // wavefronts per block
// Largest token count routed here (Wup 14336 x 4096, one token: FP6G 51 ->
// 21 us, AUTOFP8 58 -> 28 us, AUTOFP6E 56 -> 33 us against the 64-token GEMM
// tile; still ahead at 4 tokens, behind at 8, where the tile's decode of each
// weight serves every token)
constexpr int kFmtGemvTokens = 4;
// Largest b * K whose activations the variant GEMV decodes into LDS itself
// (32 KB of fp16; K <= 16384, so at most 512 mask bytes); above it, and at 3-4
// tokens, a panel pass writes them first.
constexpr int64_t kFmtXlElems = 16384;

template <int FMT, int TB, int RPW, int U, bool XL>
__global__ __launch_bounds__(64 * kFmtGemvWaves) void gemv_fmt_kernel(LinearArgs a) {
  constexpr bool F8 = FMT == AUTOFP_FMT_AUTOFP8;
  constexpr bool G6 = FMT == AUTOFP_FMT_FP6G;
  constexpr int64_t OW = F8 ? 2 : 1;   // offset bytes per refined subgroup
  constexpr uint32_t OOB = 0x80000000u;
  constexpr int NT = 64 * kFmtGemvWaves;
  __shared__ uint2 tabs[512];
  uint2 *dtab = tabs, *stab = tabs + 256;
  uint32_t *t8 = (uint32_t *)tabs;
  const int L = run_level(a);
  const bool refine_w = !G6 && (L == 6 || (F8 && L == 8)) && a.w_mask != nullptr && a.w_offsets != nullptr &&
                        a.n_refined > 0;
  if (refine_w) fill_decode_tables<FMT>(dtab, stab, L);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t K = a.k, R = a.n_refined;
  const int64_t CB = G6 ? 3 * K / 4 : K / 2;   // code bytes per weight row
  const int64_t items = K >> 5;                 // 32-element items per row

  // XL (b * K <= kFmtXlElems): the block decodes the activations into LDS
  // itself, quad-major ([token][quad q of an item][item], 16 bytes each, so
  // the lanes' reads of one quad are consecutive), and forms the weight
  // mask's exclusive popcount prefix there (pref[j]: refined subgroups before
  // item j) - no activation panel, no prefix pass.
  extern __shared__ __align__(16) unsigned char xl_lds[];
  uint4 *xs = (uint4 *)xl_lds;
  int32_t *pref = (int32_t *)(xl_lds + (XL ? a.b * K * 2 : 0));
  if constexpr (XL) {
    constexpr int PER = kFmtXlElems / 8 / NT;   // 8-element activation items per thread
    const bool refine_x = !G6 && (L == 6 || (F8 && L == 8)) && a.x_offsets != nullptr;
    const uint32_t per_row = (uint32_t)(K >> 3), nx = (uint32_t)a.b * per_row;
    uint4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t e = threadIdx.x + (uint32_t)(i * NT);
      const uint32_t t = e / per_row, k0 = (e - t * per_row) * 8;
      v[i] = e < nx ? act_decode8_fmt(a, t, k0, refine_x, L) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t e = threadIdx.x + (uint32_t)(i * NT);
      const uint32_t t = e / per_row, k0 = (e - t * per_row) * 8;
      if (e < nx) xs[(t * 4 + ((k0 >> 3) & 3)) * items + (k0 >> 5)] = v[i];
    }
    if (refine_w) {
      // items <= 512: thread t takes mask bytes 2t and 2t + 1
      const uint32_t m0 = 2 * threadIdx.x < items ? a.w_mask[2 * threadIdx.x] : 0u;
      const uint32_t m1 = 2 * threadIdx.x + 1 < items ? a.w_mask[2 * threadIdx.x + 1] : 0u;
      const int32_t own = __popc(m0) + __popc(m1);
      int32_t inc = own;   // inclusive scan over the wavefront
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(inc, o, 64);
        inc += lane >= o ? y : 0;
      }
      __shared__ int32_t wsum[kFmtGemvWaves];
      if (lane == 63) wsum[wave] = inc;
      __syncthreads();
      int32_t ex = inc - own;
      for (int w = 0; w < wave; ++w) ex += wsum[w];
      if (2 * threadIdx.x < items) pref[2 * threadIdx.x] = ex;
      if (2 * threadIdx.x + 1 < items) pref[2 * threadIdx.x + 1] = ex + __popc(m0);
    }
  }
  __syncthreads();
  const int64_t n0 = ((int64_t)blockIdx.x * kFmtGemvWaves + wave) * RPW;
  if (n0 >= a.n) return;
  const int64_t nrows = (a.n - n0) < RPW ? (a.n - n0) : RPW;
  // this wavefront's rows only, so offsets stay 32-bit; rows past n, and
  // items past K, read as zero
  const __amdgpu_buffer_rsrc_t rc = rsrc(a.w_codes + n0 * CB, nrows * CB);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.w_scales + n0 * (K >> 4), nrows * (K >> 4));
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(refine_w ? a.w_offsets + n0 * R * OW : a.w_codes, refine_w ? nrows * R * OW + 16 : 0);
  const __amdgpu_buffer_rsrc_t rm = rsrc(refine_w ? a.w_mask : a.w_codes, refine_w ? items : 0);
  const __amdgpu_buffer_rsrc_t rp =
      rsrc(refine_w && !XL ? (const void *)a.prefix : a.w_codes, refine_w && !XL ? 4 * items : 0);
  // !XL: activation panel [b][kpad] fp16 (b <= TB <= 4): tokens past b read as zero
  const __amdgpu_buffer_rsrc_t rx = rsrc(XL ? (const void *)a.w_codes : (const void *)a.xh, XL ? 0 : a.b * a.kpad * 2);

  float acc[RPW][TB];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[r][t] = 0.0f;

  // U items per lane per pass (items jb, jb + 64, ...), every load of the
  // pass issued before the first use: mask bytes and prefixes first (the
  // offsets' positions), then activations, codes and scales, then offsets
  for (int64_t jb = lane; jb < items; jb += 64 * U) {
    uint32_t mb[U], joff[U];
    int32_t pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = jb + 64 * u;
      joff[u] = j < items ? (uint32_t)j : OOB;
      mb[u] = 0;
      pos[u] = 0;
      if (refine_w) {
        mb[u] = __builtin_amdgcn_raw_buffer_load_b8(rm, (int)joff[u], 0, 0);
        if constexpr (XL) pos[u] = j < items ? pref[j] : 0;
        else pos[u] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (int)(j < items ? 4 * joff[u] : OOB), 0, 0);
      }
    }
    half8v xv[U][TB][4];
    u32x4v c[U][RPW];
    u32x2v cx[U][RPW];
    uint32_t s2[U][RPW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = joff[u] != OOB;
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (XL) {
            xv[u][t][q] = live && t < a.b ? __builtin_bit_cast(half8v, xs[(t * 4 + q) * items + joff[u]])
                                          : half8v{};
          } else {
            const uint32_t off = live && t < a.b ? (uint32_t)((t * a.kpad + 32 * joff[u] + 8 * q) * 2) : OOB;
            xv[u][t][q] = __builtin_bit_cast(half8v, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
          }
        }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if constexpr (G6) {
          const uint32_t off = live ? (uint32_t)(r * CB + 24 * joff[u]) : OOB;
          c[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)off, 0, 0);
          cx[u][r] = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)(live ? off + 16 : OOB), 0, 0);
        } else {
          c[u][r] = __builtin_amdgcn_raw_buffer_load_b128(
              rc, (int)(live ? (uint32_t)(r * (K >> 1) + 16 * joff[u]) : OOB), 0, 0);
          cx[u][r] = u32x2v{0u, 0u};
        }
        s2[u][r] = __builtin_amdgcn_raw_buffer_load_b16(
            rs, (int)(live ? (uint32_t)(r * (K >> 4) + 2 * joff[u]) : OOB), 0, 0);
      }
    }
    u32x3v o[U][RPW];
    u32x4v o4[U][RPW];
    uint32_t o5[U][RPW], sh[U][RPW];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        o[u][r] = u32x3v{0u, 0u, 0u};
        o4[u][r] = u32x4v{0u, 0u, 0u, 0u};
        o5[u][r] = 0;
        sh[u][r] = 0;
        if (refine_w) {
          const int64_t p = (r * R + pos[u]) * OW;   // byte of the item's first offset
          const uint32_t al = (uint32_t)(p & ~(int64_t)3);
          sh[u][r] = (uint32_t)(p & 3);
          if constexpr (F8) {
            o4[u][r] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)al, 0, 0);
            o5[u][r] = __builtin_amdgcn_raw_buffer_load_b32(ro, (int)(al + 16), 0, 0);
          } else {
            o[u][r] = __builtin_amdgcn_raw_buffer_load_b96(ro, (int)al, 0, 0);
          }
        }
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        half8v h[4];
        decode_w32<FMT, true>(c[u][r], cx[u][r], s2[u][r], o[u][r], o4[u][r], o5[u][r], mb[u], sh[u][r], L,
                              refine_w, dtab, stab, t8, h);
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][t] = dot8(h[q], xv[u][t][q], acc[r][t]);
      }
  }

  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
  const bool out_bf16 = a.y_dtype == AUTOFP_BF16;
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const float v = wave_sum_f(acc[r][t]) * scale;
      if (lane == r * TB + t && r < nrows && t < a.b) {
        const int64_t i = (int64_t)t * a.n + n0 + r;
        if (out_bf16) ((uint16_t *)a.y)[i] = f32_to_bf16_rne(v);
        else ((float *)a.y)[i] = v;
      }
    }
}

// The variant GEMV stages the activations and the mask prefix in LDS itself
// at 1-2 tokens, where each block's redundant activation decode is at most a
// quarter of its weight decode (4 wavefronts x 2 rows; Wup one token: FP6G
// 21.8 -> 18.6 us, AUTOFP8 30.1 -> 25.9 us). At 4 tokens (one row per
// wavefront) it would match the weight decode: 53 -> 71 us.
bool fmt_gemv_xl(const LinearArgs &a) { return a.b <= 2 && a.b * a.k <= kFmtXlElems; }

template <int FMT, int TB>
hipError_t launch_gemv_fmt_t(const LinearArgs &a, hipStream_t s) {
  constexpr int RPW = TB <= 2 ? 2 : 1;   // weight rows per wavefront
  constexpr int U = 1;                   // items per lane per pass
  const int64_t rows_per_block = (int64_t)kFmtGemvWaves * RPW;
  const dim3 grid((unsigned)((a.n + rows_per_block - 1) / rows_per_block)), block(64 * kFmtGemvWaves);
  if (fmt_gemv_xl(a)) {
    const size_t lds = (size_t)(a.b * a.k * 2 + 4 * (a.k / 32 + 1));
    hipLaunchKernelGGL((gemv_fmt_kernel<FMT, TB, RPW, U, true>), grid, block, lds, s, a);
  } else {
    hipLaunchKernelGGL((gemv_fmt_kernel<FMT, TB, RPW, U, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemv_fmt(const LinearArgs &a, hipStream_t s) {
  if (a.b <= 1) return launch_gemv_fmt_t<FMT, 1>(a, s);
  if (a.b <= 2) return launch_gemv_fmt_t<FMT, 2>(a, s);
  return launch_gemv_fmt_t<FMT, 4>(a, s);
}

}  // namespace

bool gemm_small_m_ok(const LinearArgs &a) { return a.k % kBK2 == 0; }

// 64 tokens x 256 rows per block: the batched-decode path (17..64 tokens per
// launch), where the weight stream bounds the time and every decoded weight
// tile serves all tokens from LDS.
hipError_t launch_gemm_small_m(const LinearArgs &a, hipStream_t s) {
  const int64_t mtiles = (a.b + 63) / 64;
  if (mtiles * ((a.n + 255) / 256) >= 256) {
    const size_t lds = 2 * (size_t)(64 * kBK2 * 2 + 256 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 256, kDecodeWaves>), dim3((unsigned)(mtiles * ((a.n + 255) / 256))),
                       dim3(64 * kDecodeWaves), lds, s, a);
  } else if (mtiles * ((a.n + 127) / 128) >= 256) {
    // narrower tiles when 256-row tiles leave CUs idle (28672 x 8192 at 64
    // tokens: 161 us at 256 rows, 122 at 128, 114 at 64)
    const size_t lds = 2 * (size_t)(64 * kBK2 * 2 + 128 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 128, kDecodeWaves>), dim3((unsigned)(mtiles * ((a.n + 127) / 128))),
                       dim3(64 * kDecodeWaves), lds, s, a);
  } else if (mtiles * ((a.n + 63) / 64) >= 256) {
    // two wavefront groups over K (28672 x 8192 at 64 tokens: 126 -> 102 us;
    // four groups: 118 us)
    const size_t lds = 2 * 2 * (size_t)(64 * kBK2 * 2 + 64 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 64, 4, 2>), dim3((unsigned)(mtiles * ((a.n + 63) / 64))),
                       dim3(64 * 4 * 2), lds, s, a);
  } else {
    const size_t lds = 4 * 2 * (size_t)(64 * kBK2 * 2 + 64 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 64, 4, 4>), dim3((unsigned)(mtiles * ((a.n + 63) / 64))),
                       dim3(64 * 4 * 4), lds, s, a);
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemm_fmt_t(const LinearArgs &a, hipStream_t s) {
  if (a.b <= kFmtGemvTokens) return launch_gemv_fmt<FMT>(a, s);
  const int64_t nt256 = (a.n + 255) / 256;
  if (a.b >= 128) {
    const int64_t mtiles = (a.b + kBM2 - 1) / kBM2;
    // AUTOFP8 decodes on 128-row tiles (256 rows would exceed 128 VGPRs)
    const bool alt = a.k <= kAltMaxK;
    if constexpr (FMT != AUTOFP_FMT_AUTOFP8) {
      if (mtiles * nt256 >= 256) {
        const size_t lds = 2 * (size_t)(kBM2 * kBK2 * 2 + 256 * kBK2 * 2) + kTabBytes;
        if (alt)
          hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 256, kGemmWaves, 1, FMT, true>), dim3((unsigned)(mtiles * nt256)),
                             dim3(64 * kGemmWaves), lds, s, a);
        else
          hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 256, kGemmWaves, 1, FMT>), dim3((unsigned)(mtiles * nt256)),
                             dim3(64 * kGemmWaves), lds, s, a);
        return hipGetLastError();
      }
    }
    const size_t lds = 2 * (size_t)(kBM2 * kBK2 * 2 + 128 * kBK2 * 2) + kTabBytes;
    if (alt)
      hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 128, kGemmWaves, 1, FMT, true>),
                         dim3((unsigned)(mtiles * ((a.n + 127) / 128))), dim3(64 * kGemmWaves), lds, s, a);
    else
      hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 128, kGemmWaves, 1, FMT>),
                         dim3((unsigned)(mtiles * ((a.n + 127) / 128))), dim3(64 * kGemmWaves), lds, s, a);
    return hipGetLastError();
  }
  const int64_t mtiles = (a.b + 63) / 64;
  if (mtiles * nt256 >= 256) {
    const size_t lds = 2 * (size_t)(64 * kBK2 * 2 + 256 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 256, kDecodeWaves, 1, FMT>), dim3((unsigned)(mtiles * nt256)),
                       dim3(64 * kDecodeWaves), lds, s, a);
  } else {
    const size_t lds = 4 * 2 * (size_t)(64 * kBK2 * 2 + 64 * kBK2 * 2) + kTabBytes;
    hipLaunchKernelGGL((gemm_lds_kernel<64, 64, 4, 4, FMT>), dim3((unsigned)(mtiles * ((a.n + 63) / 64))),
                       dim3(64 * 4 * 4), lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_fmt(const LinearArgs &a, hipStream_t s) {
  if (a.fmt != AUTOFP_FMT_AUTOFP6 && !fmt_gemv_xl(a)) {
    // the fp16 activation panel and (offset formats, refined weight) the
    // mask prefix the tiles and the panel GEMV read
    hipError_t e = launch_act_dequant(a, s);
    if (e != hipSuccess) return e;
    if (a.fmt != AUTOFP_FMT_FP6G && a.w_mask) {
      e = launch_mask_prefix(a.w_mask, mask_bytes(a.k), a.prefix, s);
      if (e != hipSuccess) return e;
    }
  }
  switch (a.fmt) {
    case AUTOFP_FMT_AUTOFP6E: return launch_gemm_fmt_t<AUTOFP_FMT_AUTOFP6E>(a, s);
    case AUTOFP_FMT_AUTOFP8: return launch_gemm_fmt_t<AUTOFP_FMT_AUTOFP8>(a, s);
    case AUTOFP_FMT_FP6G: return launch_gemm_fmt_t<AUTOFP_FMT_FP6G>(a, s);
    default: return launch_gemm(a, s);
  }
}

hipError_t launch_gemm(const LinearArgs &a, hipStream_t s) {
  if (a.k % kBK2 == 0 && a.b >= 128) {
    // 256 x 256 tiles when they still give every CU a block, else 256 x 128
    const int64_t mtiles = (a.b + kBM2 - 1) / kBM2;
    const int64_t big = mtiles * ((a.n + 255) / 256);
    const bool alt = a.k <= kAltMaxK;
    if (big >= 256) {
      const size_t lds = 2 * (size_t)(kBM2 * kBK2 * 2 + 256 * kBK2 * 2) + kTabBytes;
      if (alt)
        hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 256, kGemmWaves, 1, AUTOFP_FMT_AUTOFP6, true>), dim3((unsigned)big),
                           dim3(64 * kGemmWaves), lds, s, a);
      else
        hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 256, kGemmWaves>), dim3((unsigned)big), dim3(64 * kGemmWaves), lds,
                           s, a);
    } else {
      const size_t lds = 2 * (size_t)(kBM2 * kBK2 * 2 + 128 * kBK2 * 2) + kTabBytes;
      if (alt)
        hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 128, kGemmWaves, 1, AUTOFP_FMT_AUTOFP6, true>),
                           dim3((unsigned)(mtiles * ((a.n + 127) / 128))), dim3(64 * kGemmWaves), lds, s, a);
      else
        hipLaunchKernelGGL((gemm_lds_kernel<kBM2, 128, kGemmWaves>), dim3((unsigned)(mtiles * ((a.n + 127) / 128))),
                           dim3(64 * kGemmWaves), lds, s, a);
    }
    return hipGetLastError();
  }
  if (a.k % kBK2 == 0) return launch_gemm_small_m(a, s);
  const int64_t mtiles = (a.b + BM - 1) / BM;
  const int64_t ntiles = (a.n + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(mtiles * ntiles)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace afp
