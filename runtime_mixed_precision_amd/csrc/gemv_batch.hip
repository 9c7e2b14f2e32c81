// Batched decode GEMV (up to 64 tokens per launch) and per-token precision
// levels for gfx950.
//
// "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
// Exponent-Mantissa Refinement" (arXiv 2611.10165v1), §3.1-3.2 (levels 2, 4,
// 6 and the refined product), §4 (the linear layer on packed operands) and
// §4.2 "Serving Mixed-Precision Batches" (requests of one batch at different
// levels served by one GEMM over the union of their refinements, Fig. 6).
//
// Result: y[t][n] = sum_k What_l(t)[n][k] * Xhat_l(t)[t][k], where l(t) is the
// level of token t (one level for the whole call, or one per token). Decoded
// operands without their tensor scales are exact in fp16 (at most 10
// significant bits), so v_mfma_f32_16x16x32_f16 forms exact products and
// only the fp32 accumulation rounds; T_W * T_X (times c for a level-2 token)
// is applied once per output.
//
// Work split. A block of 4 wavefronts owns 16 NF weight rows (NF = 4, or 2
// above 32 tokens with per-token levels) and 16 TT tokens (TT = 1, 2 or 4
// tiles of 16); the wavefronts split the block's K range into four contiguous
// parts, and the blocks of one row tile split K into S parts (S > 1 only
// when the row tiles alone leave compute units idle). Per 128-element K step
// a lane (r16 = l % 16,
// q = l / 16) loads, straight into registers, elements 32q .. 32q + 31 of
// weight rows 16f + r16 and of tokens 16tt + r16 (one 16-byte load each) and,
// at level 6, the 12-byte window of the row's compacted weight offsets and the
// token's eight activation offset bytes. The E4M3 scales of the wavefront's
// rows and tokens over its whole K range go to LDS once, with 8-byte loads, so
// the loop issues only the code (and offset) loads. MFMA kk (0..3) of a step
// takes, in K slot q, the lane's elements 32q + 8kk .. +7 of both operands:
// the same K permutation on both sides. Loads run two steps ahead of the
// arithmetic (one with level-6 operands).
//
// The 4 wavefronts' accumulators are added through LDS in wavefront order;
// with S > 1 the block writes its fp32 partial tile to the workspace and a
// second kernel adds the S partials in split order (deterministic, no
// atomics) and applies the scale.
//
// Mixed levels (§4.2): with per-token levels, a step decodes the weight
// fragment once per level present among the block's tokens (AutoFP2 digits
// at 2, NVFP4 at 4, refined at 6) and runs that level's MFMAs with the
// activation rows of tokens at other levels set to zero - the union of the
// levels' work, each token seeing only its own level. A token at level 6
// reads its own refined activation (its mask M_A and offsets).
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

constexpr int kBW = 4;           // wavefronts per block (K groups)
constexpr int kStep = 128;       // K elements per step
constexpr int kMaxBlockSteps = 64;     // K steps per block (LDS copies of the scales and the mask plan)
constexpr int kWaveSteps = kMaxBlockSteps / kBW;   // K steps per wavefront at most
constexpr int kScaleRow = 8 * kWaveSteps;          // LDS bytes of one row's scales per wavefront
constexpr size_t kTabBytes = 2 * 256 * 8 + 4 * kMaxBlockSteps * (1 + 4);
constexpr uint32_t kOOBb = 0x80000000u;
constexpr int kPartFloats = 32768;     // partial-tile floats per token (S * N bound)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

__device__ __forceinline__ half8v h8(uint4 v) { return __builtin_bit_cast(half8v, v); }

// E4M3 scale code (low byte of c, sign ignored) to fp16, exact and branch-free:
// a normal code e|m is 2^(e-7)(1 + m/8), fp16 bits ((e + 8) << 10) | (m << 7)
// = (code << 7) + 0x2000; a subnormal m * 2^-9 is a normal fp16 value.
__device__ __forceinline__ _Float16 e4m3_half(uint32_t c) {
  const uint32_t code = c & 0x7Fu;
  const _Float16 hn = __builtin_bit_cast(_Float16, (uint16_t)((code << 7) + 0x2000u));
  const _Float16 hs = (_Float16)(code & 7u) * (_Float16)0.001953125f;
  return (code >> 3) ? hn : hs;
}

// fp16 decode of 8 activation elements (one code dword) with their group
// scale byte and, when REF, their two offset bytes (zero when unrefined):
// B * (q + d/8).
template <bool REF>
__device__ __forceinline__ half8v act8(uint32_t cw, uint32_t sbyte, uint32_t ob) {
  half8v h = fp4x8_to_half8(cw);
  if (REF) {
    const uint2 d0 = delta_words(ob & 0xFFu), d1 = delta_words((ob >> 8) & 0xFFu);
    h += h8(make_uint4(d0.x, d0.y, d1.x, d1.y));
  }
  return h * e4m3_half(sbyte);
}

template <int TT, int NF>
struct StepRegs {
  u32x4v wc[NF];     // weight codes: 32 elements of a row per fragment
  u32x3v wo[NF];     // level 6: offset windows
  u32x4v xc[TT];     // activation codes per 16-token tile
  u32x2v xo[TT];     // eight activation offset bytes per token tile
};

// TT: 16-token tiles (1, 2 or 4); NF: 16-row weight fragments per wavefront
// (the block's rows: 16 NF). MIXED: per-token levels from a.bits_rows.
// REF: a level-6 token may occur (host level 6, a device-side level or
// per-token levels); every step then issues the offset loads too, with an
// out-of-range offset (no memory access, zeros) where they are not needed,
// so each step issues the same loads and the waits stay exact.
//
// Lane l = (r16 = l % 16, q = l / 16): in a 128-element step it holds
// elements 32q .. 32q + 31 of weight rows 16f + r16 (f < NF) and of tokens
// 16tt + r16, so the 4 lanes of a row read 64 contiguous bytes of it per
// load. MFMA kk (v_mfma_f32_16x16x32_f16, K slot q) takes the lane's
// elements 32q + 8kk .. +7 of both operands.
template <int TT, int NF, bool MIXED, bool REF>
__global__ __launch_bounds__(64 * kBW) __attribute__((amdgpu_waves_per_eu(2))) void gemv_batch_kernel(LinearArgs a) {
  constexpr int PD = REF ? 1 : 2;   // steps of loads in flight ahead of the arithmetic
  constexpr int kBRows = 16 * NF;
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // uniform: scalar loop bounds
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int64_t K = a.k;
  const int64_t nrb = (a.n + kBRows - 1) / kBRows;
  const int64_t rb = blockIdx.x % nrb;
  const int split = (int)(blockIdx.x / nrb);
  const int64_t n0 = rb * kBRows;
  const int64_t nst = K / kStep;
  const int64_t bs0 = nst * split / a.splits, bs1 = nst * (split + 1) / a.splits;
  const int64_t nsb = bs1 - bs0;
  const int64_t ws0 = bs0 + nsb * wave / kBW, ws1 = bs0 + nsb * (wave + 1) / kBW;

  // levels present in this call (uniform over the block)
  int tlev[TT];
  uint32_t present;
  if (MIXED) {
    uint32_t p = 0;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int64_t t = 16 * tt + r16;
      tlev[tt] = t < a.b ? a.bits_rows[t] : 0;
      p |= tlev[tt] == 2 ? 1u : tlev[tt] == 4 ? 2u : tlev[tt] == 6 ? 4u : 0u;
    }
    // OR over the wavefront (every wavefront sees every token)
    present = (__ballot(p & 1u) ? 1u : 0u) | (__ballot(p & 2u) ? 2u : 0u) | (__ballot(p & 4u) ? 4u : 0u);
  } else {
    const int L = a.bits_dev ? *a.bits_dev : a.bits;
    present = L == 2 ? 1u : L == 6 ? 4u : 2u;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) tlev[tt] = L;
  }
  const bool any6 = (present & 4u) != 0;
  const bool refine_w = REF && any6 && a.w_mask != nullptr && a.w_offsets != nullptr && a.n_refined > 0;
  const bool refine_x = REF && any6 && a.x_offsets != nullptr;
  const int64_t R = a.n_refined;

  // LDS: level-6 decode tables and this block's slice of the mask plan (one
  // mask byte and prefix entry per 32 elements)
  uint2 *dtab = (uint2 *)lds;
  uint2 *stab = dtab + 256;
  uint8_t *pl_mask = (uint8_t *)(stab + 256);                    // [4 * nsb] mask bytes
  int32_t *pl_pos = (int32_t *)(pl_mask + 4 * kMaxBlockSteps);     // [4 * nsb] prefix entries
  if (refine_w) {
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
    // the slice's mask bytes and their exclusive popcount prefix (refined
    // subgroups before each byte), formed here: mask dword d holds the 4 mask
    // bytes of step d (128 elements); thread t counts the refined subgroups of
    // a contiguous run of the dwords before the slice's end (at most two per
    // thread for K <= 65536, the largest K whose masks the library selects),
    // the counts are scanned across the block (wavefront scans, then the
    // wavefront totals in order) and each thread writes the slice entries of
    // its run.
    const uint32_t *m32 = (const uint32_t *)a.w_mask;
    const int64_t nd = bs0 + nsb;
    const int64_t rd = (nd + 64 * kBW - 1) / (64 * kBW);
    const int64_t d0 = (int64_t)threadIdx.x * rd;
    const int64_t d1 = (d0 + rd) < nd ? (d0 + rd) : nd;
    int32_t own = 0;
    for (int64_t d = d0; d < d1; ++d) own += __popc(m32[d]);
    int32_t inc = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(inc, o, 64);
      inc += lane >= o ? y : 0;
    }
    __shared__ int32_t wtot[kBW];
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    int32_t pos = inc - own;
    for (int w = 0; w < wave; ++w) pos += wtot[w];
    for (int64_t d = d0; d < d1; ++d) {
      const uint32_t m = m32[d];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t mb = (m >> (8 * e)) & 0xFFu;
        if (d >= bs0) {
          pl_mask[4 * (d - bs0) + e] = (uint8_t)mb;
          pl_pos[4 * (d - bs0) + e] = pos;
        }
        pos += __popc(mb);
      }
    }
  }
  __syncthreads();

  // buffer resources: the block's weight rows, all tokens' activations
  const int64_t nrows = (a.n - n0) < kBRows ? (a.n - n0) : kBRows;
  const __amdgpu_buffer_rsrc_t rc = rsrc_b(a.w_codes + n0 * (K >> 1), nrows * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = rsrc_b(a.w_scales + n0 * (K >> 4), nrows * (K >> 4));
  const __amdgpu_buffer_rsrc_t ro =
      rsrc_b(refine_w ? a.w_offsets + n0 * R : a.w_codes, refine_w ? nrows * R + 16 : 0);
  const __amdgpu_buffer_rsrc_t rxc = rsrc_b(a.x_codes, a.b * (K >> 1));
  const __amdgpu_buffer_rsrc_t rxs = rsrc_b(a.x_scales, a.b * (K >> 4));
  const __amdgpu_buffer_rsrc_t rxo = rsrc_b(refine_x ? a.x_offsets : a.x_codes, refine_x ? a.b * (K >> 2) : 0);

  // the wavefront's E4M3 scales (its weight rows and tokens over its K range)
  // go to LDS once, with 8-byte loads (one step of a row each), so the loop
  // issues only the 16-byte code loads: [16 NF rows][kScaleRow], then
  // [16 TT tokens][kScaleRow]
  unsigned char *scl = lds + kTabBytes + (size_t)wave * (16 * (NF + TT)) * kScaleRow;
  const int nsw = (int)(ws1 - ws0);
  {
    constexpr int UW = (16 * NF * kWaveSteps) / 64, UX = (16 * TT * kWaveSteps) / 64;
    u32x2v sw[UW], sx[UX];
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int u = lane + 64 * i, row = u / kWaveSteps, j = u % kWaveSteps;
      const uint32_t off = j < nsw ? (uint32_t)(row * (K >> 4) + 8 * (ws0 + j)) : kOOBb;
      sw[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int u = lane + 64 * i, t = u / kWaveSteps, j = u % kWaveSteps;
      const uint32_t off = j < nsw ? (uint32_t)(t * (K >> 4) + 8 * (ws0 + j)) : kOOBb;
      sx[i] = __builtin_amdgcn_raw_buffer_load_b64(rxs, (int)off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int u = lane + 64 * i;
      *(u32x2v *)(scl + (u / kWaveSteps) * kScaleRow + 8 * (u % kWaveSteps)) = sw[i];
    }
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int u = lane + 64 * i;
      *(u32x2v *)(scl + (16 * NF + u / kWaveSteps) * kScaleRow + 8 * (u % kWaveSteps)) = sx[i];
    }
  }
  // LDS byte offsets of the lane's two scale bytes of its first step
  uint32_t wsl[NF], xsl[TT];
#pragma unroll
  for (int f = 0; f < NF; ++f) wsl[f] = (uint32_t)((16 * f + r16) * kScaleRow + 2 * q);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) xsl[tt] = (uint32_t)((16 * (NF + tt) + r16) * kScaleRow + 2 * q);

  // per-lane byte offsets of element 32q of step 0 (32-bit: every buffer is
  // below 2^31 bytes), then + st * (bytes per step). A lane whose token is past
  // the batch, or whose row is past the weight, falls outside its buffer's
  // range and reads zeros. kOOBb added to a base keeps every step of it out of
  // range (an unrefined token's offsets).
  const uint32_t kb2 = (uint32_t)(K >> 1), kb4 = (uint32_t)(K >> 2);
  uint32_t wcb[NF], wob[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const uint32_t row = (uint32_t)(16 * f + r16);
    wcb[f] = row * kb2 + 16u * q;
    wob[f] = row * (uint32_t)R;
  }
  bool xref[TT];   // this lane's token reads refined activations
  uint32_t xcb[TT], xob[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const uint32_t t = (uint32_t)(16 * tt + r16);
    xref[tt] = refine_x && tlev[tt] == 6;
    xcb[tt] = t * kb2 + 16u * q;
    xob[tt] = (t * kb4 + 8u * q) + (xref[tt] ? 0u : kOOBb);
  }

  auto load = [&](int64_t st, StepRegs<TT, NF> &g) {
    // steps past this wavefront's range (the prefetch tail) read nothing
    const uint32_t kill = st < ws1 ? 0u : kOOBb;
    const uint32_t s64 = (uint32_t)st * 64u + kill;
    int32_t pos = 0;
    if (REF && refine_w) pos = pl_pos[4 * (st - bs0) + q];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      g.wc[f] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(wcb[f] + s64), 0, 0);
      if (REF) {
        const uint32_t al = ((wob[f] + (uint32_t)pos) & ~3u) + (refine_w ? kill : kOOBb);
        g.wo[f] = __builtin_amdgcn_raw_buffer_load_b96(ro, (int)al, 0, 0);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      g.xc[tt] = __builtin_amdgcn_raw_buffer_load_b128(rxc, (int)(xcb[tt] + s64), 0, 0);
      if (REF) g.xo[tt] = __builtin_amdgcn_raw_buffer_load_b64(rxo, (int)(xob[tt] + (uint32_t)st * 32u + kill), 0, 0);
    }
  };

  float4v acc[NF][TT];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[f][tt] = float4v{0.f, 0.f, 0.f, 0.f};

  // weight fragment f of a step at level `lev`, dword kk (8 elements)
  auto wfrag = [&](const StepRegs<TT, NF> &g, int f, int kk, int lev, const uint32_t (&E)[2], uint32_t ws) -> half8v {
    uint32_t c = g.wc[f][kk];
    if (lev == 2) c = autofp2_codes(c);
    half8v v = fp4x8_to_half8(c);
    if (lev == 6 && refine_w) {
      const uint2 de = dtab[(E[kk >> 1] >> (16 * (kk & 1))) & 0xFFu];
      const uint2 dd = dtab[(E[kk >> 1] >> (16 * (kk & 1) + 8)) & 0xFFu];
      v += h8(make_uint4(de.x, de.y, dd.x, dd.y));
    }
    return v * e4m3_half(ws >> (8 * (kk >> 1)));
  };

  auto compute = [&](int64_t st, const StepRegs<TT, NF> &g) {
    // this step's scale bytes from LDS
    const uint32_t so = (uint32_t)(8 * (st - ws0));
    uint32_t wsc[NF], xsc[TT];
#pragma unroll
    for (int f = 0; f < NF; ++f) wsc[f] = *(const uint16_t *)(scl + wsl[f] + so);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) xsc[tt] = *(const uint16_t *)(scl + xsl[tt] + so);
    // level-6 offset bytes of the lane's 8 subgroups, per fragment
    uint32_t E[NF][2];
#pragma unroll
    for (int f = 0; f < NF; ++f) E[f][0] = E[f][1] = 0;
    if (refine_w) {
      const uint32_t m = pl_mask[4 * (st - bs0) + q];
      const int32_t pos = pl_pos[4 * (st - bs0) + q];
      const uint2 sel = stab[m];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint32_t sh = (wob[f] + (uint32_t)pos) & 3u;
        const uint32_t lo = __builtin_amdgcn_alignbyte(g.wo[f][1], g.wo[f][0], sh);
        const uint32_t hi = __builtin_amdgcn_alignbyte(g.wo[f][2], g.wo[f][1], sh);
        E[f][0] = __builtin_amdgcn_perm(hi, lo, sel.x);
        E[f][1] = __builtin_amdgcn_perm(hi, lo, sel.y);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half8v xa[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint32_t ob = REF ? (g.xo[tt][kk >> 1] >> (16 * (kk & 1))) : 0u;
        xa[tt] = act8<REF>(g.xc[tt][kk], xsc[tt] >> (8 * (kk >> 1)), ob);
      }
#pragma unroll
      for (int li = 0; li < 3; ++li) {
        const int lev = 2 + 2 * li;
        if (!(present & (1u << li))) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const half8v wf = wfrag(g, f, kk, lev, E[f], wsc[f]);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            half8v x = xa[tt];
            if (MIXED && tlev[tt] != lev) x = half8v{0, 0, 0, 0, 0, 0, 0, 0};
            acc[f][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, x, acc[f][tt], 0, 0, 0);
          }
        }
      }
    }
  };

  // main loop: a ring of PD + 1 register stages, loads PD steps ahead
  StepRegs<TT, NF> ring[PD + 1];
#pragma unroll
  for (int u = 0; u < PD; ++u) load(ws0 + u, ring[u]);
  for (int64_t st = ws0; st < ws1; st += PD + 1) {
#pragma unroll
    for (int u = 0; u < PD + 1; ++u) {
      load(st + u + PD, ring[(u + PD) % (PD + 1)]);
      if (st + u < ws1) compute(st + u, ring[u]);
    }
  }

  // K groups: wavefronts 1..3 leave their accumulators in LDS (lane-minor),
  // wavefront 0 adds them in wavefront order
  __syncthreads();
  float *red = (float *)lds;
  constexpr int PER = NF * TT * 4;
  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(((wave - 1) * PER) + (f * TT + tt) * 4 + v) * 64 + lane] = acc[f][tt][v];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll 1
  for (int g = 1; g < kBW; ++g)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][tt][v] += red[(((g - 1) * PER) + (f * TT + tt) * 4 + v) * 64 + lane];

  // D (fragment f, token tile tt): lane holds token 16 tt + lane % 16 and
  // weight rows n0 + 16 f + 4 (lane / 16) + v
  const float tw = (*a.w_T) * (*a.x_T);
  const bool out_bf16 = a.y_dtype == AUTOFP_BF16;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int64_t t = 16 * tt + r16;
    if (t >= a.b) continue;
    const int lev = MIXED ? a.bits_rows[t] : (a.bits_dev ? *a.bits_dev : a.bits);
    const float sc = lev == 2 ? tw * a.c2 : tw;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int64_t nb = n0 + 16 * f + 4 * q;
      if (a.splits > 1) {
        float *dst = a.part + ((int64_t)split * a.b + t) * a.n;
        if (nb + 3 < a.n && (a.n & 3) == 0) {
          *(float4v *)(dst + nb) = acc[f][tt];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (nb + v < a.n) dst[nb + v] = acc[f][tt][v];
        }
      } else if (out_bf16) {
        uint16_t *y = (uint16_t *)a.y + t * a.n;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (nb + v < a.n) y[nb + v] = f32_to_bf16_rne(acc[f][tt][v] * sc);
      } else {
        float *y = (float *)a.y + t * a.n;
        if (nb + 3 < a.n && (a.n & 3) == 0) {
          *(float4v *)(y + nb) = acc[f][tt] * sc;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (nb + v < a.n) y[nb + v] = acc[f][tt][v] * sc;
        }
      }
    }
  }
}

// Sum of the S partial tiles in split order, the scale, the output dtype.
template <bool MIXED>
__global__ __launch_bounds__(256) void gemv_batch_reduce_kernel(LinearArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.b * a.n) return;
  const int64_t t = i / a.n;
  float s = a.part[i];
  for (int sp = 1; sp < a.splits; ++sp) s += a.part[(int64_t)sp * a.b * a.n + i];
  const int lev = MIXED ? a.bits_rows[t] : (a.bits_dev ? *a.bits_dev : a.bits);
  const float tw = (*a.w_T) * (*a.x_T);
  const float val = s * (lev == 2 ? tw * a.c2 : tw);
  if (a.y_dtype == AUTOFP_BF16) ((uint16_t *)a.y)[i] = f32_to_bf16_rne(val);
  else ((float *)a.y)[i] = val;
}

// K splits across blocks: enough blocks for the 256 compute units (two
// blocks per CU fit), at least 4 steps per wavefront, at most
// kMaxBlockSteps steps per block, and S * n within the partial buffer.
int batch_splits(int64_t n, int64_t k, int rows) {
  const int64_t nrb = (n + rows - 1) / rows;
  const int64_t nst = k / kStep;
  int s = 1;
  while (nrb * s < 256 && nst / (2 * s) >= 2 * kBW && (int64_t)(2 * s) * n <= kPartFloats) s *= 2;
  while ((nst + s - 1) / s > kMaxBlockSteps) ++s;
  return s;
}

// 16-row fragments per wavefront: 4 (64 rows per block), 2 above 32 tokens
// with per-token levels (the mixed kernel's registers: two wavefronts per
// SIMD). A single level 6 keeps 4 (64 tokens: Wgate|Wup 81 -> 62 us, Wdown
// 50 -> 45 us against 2).
int batch_frags(int64_t tokens, bool mixed) { return (tokens > 32 && mixed) ? 2 : 4; }

}  // namespace

int64_t gemv_batch_part_floats(int64_t tokens) { return (int64_t)kPartFloats * (tokens < 64 ? tokens : 64); }

bool gemv_batch_ok(const LinearArgs &a) {
  if (a.k % kStep != 0) return false;
  const bool mixed = a.bits_rows != nullptr;
  for (int64_t b : {a.b < 64 ? a.b : (int64_t)64, a.b % 64}) {
    if (b == 0) continue;
    const int s = batch_splits(a.n, a.k, 16 * batch_frags(b, mixed));
    if (s > 1 && (int64_t)s * a.n > kPartFloats) return false;
  }
  return true;
}

hipError_t launch_gemv_batch(const LinearArgs &a0, hipStream_t st) {
  const bool mixed = a0.bits_rows != nullptr;
  const bool ref = mixed || a0.bits_dev != nullptr || a0.bits == 6;
  for (int64_t t0 = 0; t0 < a0.b; t0 += 64) {
    LinearArgs a = a0;
    a.b = (a0.b - t0) < 64 ? (a0.b - t0) : 64;
    a.x_codes = a0.x_codes + t0 * (a0.k / 2);
    a.x_scales = a0.x_scales + t0 * (a0.k / 16);
    a.x_offsets = a0.x_offsets ? a0.x_offsets + t0 * (a0.k / 4) : nullptr;
    a.bits_rows = a0.bits_rows ? a0.bits_rows + t0 : nullptr;
    a.y = (char *)a0.y + t0 * a0.n * (a0.y_dtype == AUTOFP_BF16 ? 2 : 4);
    const int nf = batch_frags(a.b, mixed);
    const int S = batch_splits(a.n, a.k, 16 * nf);
    const int64_t nrb = (a.n + 16 * nf - 1) / (16 * nf);
    a.splits = S;
    const dim3 grid((unsigned)(nrb * S)), block(64 * kBW);
    const int tt = a.b <= 16 ? 1 : a.b <= 32 ? 2 : 4;
    const size_t red = (size_t)(kBW - 1) * nf * tt * 4 * 64 * sizeof(float);
    const size_t tab = kTabBytes + (size_t)kBW * 16 * (nf + tt) * kScaleRow;
    const size_t lds = red > tab ? red : tab;
#define AFP_BATCH(TT, NF, MX, RF) hipLaunchKernelGGL((gemv_batch_kernel<TT, NF, MX, RF>), grid, block, lds, st, a)
#define AFP_BATCH_TT(TT, NF)                \
    if (mixed) AFP_BATCH(TT, NF, true, true);  \
    else if (ref) AFP_BATCH(TT, NF, false, true); \
    else AFP_BATCH(TT, NF, false, false)
    if (tt == 1) { AFP_BATCH_TT(1, 4); }
    else if (tt == 2) { AFP_BATCH_TT(2, 4); }
    else if (nf == 2) { AFP_BATCH(4, 2, true, true); }
    else if (ref) { AFP_BATCH(4, 4, false, true); }
    else { AFP_BATCH(4, 4, false, false); }
#undef AFP_BATCH_TT
#undef AFP_BATCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (S > 1) {
      const dim3 rgrid((unsigned)((a.b * a.n + 255) / 256));
      if (mixed) hipLaunchKernelGGL(gemv_batch_reduce_kernel<true>, rgrid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL(gemv_batch_reduce_kernel<false>, rgrid, dim3(256), 0, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace afp
