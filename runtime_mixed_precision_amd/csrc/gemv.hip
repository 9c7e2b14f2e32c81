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
// Work split: a block of 4 wavefronts owns 16 weight rows and the whole K; each
// wavefront takes a contiguous quarter of the 128-element K chunks, so a
// 16-row x K/4 slab streams through its lanes with 16-byte loads
// (lane = row l%16, K slice l/16). Partial 16x16 tiles are summed in LDS.
//
// Activations: up to 16 tokens, every wavefront decodes the packed activation
// chunk it needs (tokens x 128 elements, 2 elements per lane per token) into a
// private LDS buffer and reads the MFMA operand from there - one kernel, no
// scratch. Above 16 tokens a separate pass decodes the activations once into
// an fp16 panel that the GEMV reads.
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

__device__ __forceinline__ int run_level(const LinearArgs &a) {
  return a.bits_dev ? *a.bits_dev : a.bits;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Weight side: 32 codes (16 B) and two scale bytes per lane per 128-K chunk
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
    for (int i = 0; i < 4; ++i) w4[i] = autofp2_codes(w4[i]);
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

// Sum the four K quarters and write y[token][row] (wave 0 only).
template <int TT>
__device__ __forceinline__ void reduce_store(const LinearArgs &a, float4v (&red)[4][TT][64],
                                             const float4v (&acc)[TT], int L, int64_t n0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < TT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  const int r = lane & 15, ks = lane >> 4;
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
// Activation panel (more than 16 tokens): xh[b][k] = fp16(B_A * (q + delta_A)),
// zero-padded to kpad. One thread per 8 elements.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void act_dequant_kernel(LinearArgs a) {
  const int64_t per_row = a.kpad / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.b * per_row) return;
  const int64_t row = idx / per_row;
  const int64_t k0 = (idx - row * per_row) * 8;
  half8v out = half8v{0, 0, 0, 0, 0, 0, 0, 0};
  if (k0 < a.k) {
    const int L = run_level(a);
    const uint32_t cw = *(const uint32_t *)(a.x_codes + row * (a.k / 2) + k0 / 2);
    half8v h = fp4x8_to_half8(cw);
    if (L == 6 && a.x_offsets) {
      const uint8_t *ob = a.x_offsets + row * (a.k / 4) + k0 / 4;
      half2v d0, d1, d2, d3;
      offsets_to_half4(ob[0], d0, d1);
      offsets_to_half4(ob[1], d2, d3);
      h += half8v{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
    }
    const _Float16 B = (_Float16)e4m3_value(a.x_scales[row * (a.k / 16) + k0 / 16]);
    out = h * B;
  }
  *(half8v *)(a.xh + row * a.kpad + k0) = out;
}

// ---------------------------------------------------------------------------
// GEMV for up to 16 tokens: packed activations staged per chunk in LDS
// ---------------------------------------------------------------------------

constexpr int kXRow = 136;   // halves per staged token row (128 + pad)

template <int U>
__global__ __launch_bounds__(256) void gemv_small_kernel(LinearArgs a) {
  __shared__ _Float16 xs[4][2][16][kXRow];
  __shared__ float4v red[4][1][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int64_t K = a.k;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int L = run_level(a);
  const bool refine_w = (L == 6) && a.w_mask != nullptr && a.w_offsets != nullptr;
  const bool refine_x = (L == 6) && a.x_offsets != nullptr;

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

  const int nstage = (int)a.b * 16;       // activation dwords (8 elements) per chunk
  float4v acc = float4v{0.f, 0.f, 0.f, 0.f};

  for (int64_t cb = c0; cb < c1; cb += U) {
    uint4 cw[U];
    uint32_t sw[U];
    uint32_t xc[U][4], xsb[U][4], xo[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      load_w(w, (c << 7) + (ks << 5), c < c1, cw[u], sw[u]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int idx = lane + 64 * m;
        const int t = idx >> 4;
        const int64_t k8 = (c << 7) + 8 * (idx & 15);
        xc[u][m] = 0;
        xsb[u][m] = 0;
        xo[u][m] = 0;
        if (c < c1 && idx < nstage && k8 < K) {
          xc[u][m] = *(const uint32_t *)(a.x_codes + t * (K >> 1) + (k8 >> 1));
          xsb[u][m] = a.x_scales[t * (K >> 4) + (k8 >> 4)];
          if (refine_x) xo[u][m] = *(const uint16_t *)(a.x_offsets + t * (K >> 2) + (k8 >> 2));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      if (c >= c1) break;
      const int buf = (int)((c - c0) & 1);
      // stage this chunk's activations: B_A * (q + delta_A) in fp16
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int idx = lane + 64 * m;
        if (idx < nstage) {
          half8v hx = fp4x8_to_half8(xc[u][m]);
          if (refine_x) {
            half2v d0, d1, d2, d3;
            offsets_to_half4(xo[u][m] & 0xFFu, d0, d1);
            offsets_to_half4(xo[u][m] >> 8, d2, d3);
            hx += half8v{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
          }
          hx *= (_Float16)e4m3_value(xsb[u][m]);
          *(half8v *)&xs[wave][buf][idx >> 4][8 * (idx & 15)] = hx;
        }
      }
      wave_lds_sync();
      half8v xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = (r < a.b) ? *(const half8v *)&xs[wave][buf][r][32 * ks + 8 * i]
                          : half8v{0, 0, 0, 0, 0, 0, 0, 0};
      half8v h[4];
      decode_w(a, w, L, refine_w, c, ks, cw[u], sw[u], pre, h);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(h[i], xv[i], acc, 0, 0, 0);
    }
  }
  const float4v accs[1] = {acc};
  reduce_store<1>(a, red, accs, L, n0);
}

// ---------------------------------------------------------------------------
// GEMV for 17..64 tokens: activations from the fp16 panel
// ---------------------------------------------------------------------------

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
  reduce_store<TT>(a, red, acc, L, n0);
}

}  // namespace

int64_t xh_kpad(int64_t k) { return round_up(k, 128); }

hipError_t launch_act_dequant(const LinearArgs &a, hipStream_t s) {
  const int64_t threads = a.b * (a.kpad / 8);
  hipLaunchKernelGGL(act_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

bool gemv_needs_panel(int64_t tokens) { return tokens > 16; }

hipError_t launch_gemv(const LinearArgs &a0, hipStream_t s) {
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
      hipLaunchKernelGGL((gemv_small_kernel<8>), grid, dim3(256), 0, s, a);
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
