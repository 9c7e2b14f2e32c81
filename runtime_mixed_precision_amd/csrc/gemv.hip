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
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

__device__ __forceinline__ int run_level(const LinearArgs &a) {
  return a.bits_dev ? *a.bits_dev : a.bits;
}

// ---------------------------------------------------------------------------
// Activation dequant: xh[b][k] = fp16(B_A * (q + delta_A)), zero-padded to kpad.
// One thread per 8 elements.
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
// GEMV main kernel
// ---------------------------------------------------------------------------

template <int TT, int U>
__global__ __launch_bounds__(256) void gemv_kernel(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int64_t K = a.k;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t row = n0 + r;
  const bool row_ok = row < a.n;
  const int L = run_level(a);
  const bool refine_w = (L == 6) && a.w_mask != nullptr && a.w_offsets != nullptr;
  const bool k32 = (K & 31) == 0;

  const int64_t nch = (K + 127) >> 7;
  const int64_t per = (nch + 3) >> 2;
  const int64_t c0 = wave * per;
  const int64_t c1 = (c0 + per < nch) ? c0 + per : nch;
  const int64_t mbytes = (K + 31) >> 5;

  const uint8_t *wcodes = a.w_codes + (row_ok ? row : 0) * (K >> 1);
  const uint8_t *wscl = a.w_scales + (row_ok ? row : 0) * (K >> 4);
  const uint8_t *woff = refine_w ? a.w_offsets + (row_ok ? row : 0) * (int64_t)a.n_refined : nullptr;

  int32_t pre = 0;   // refined subgroups of this row before the current chunk
  if (refine_w && c0 < c1) {
    // chunks before c0 are complete, so their four mask bytes exist
    for (int64_t m = 0; m < c0; ++m) pre += __popc(*(const uint32_t *)(a.w_mask + 4 * m));
  }

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
      const bool ok = (c < c1) && row_ok && ke < K;
      cw[u] = make_uint4(0, 0, 0, 0);
      sw[u] = 0;
      if (ok) {
        if (k32) {
          cw[u] = *(const uint4 *)(wcodes + (ke >> 1));
          sw[u] = *(const uint16_t *)(wscl + (ke >> 4));
        } else {
          const uint2 lo = *(const uint2 *)(wcodes + (ke >> 1));
          cw[u].x = lo.x;
          cw[u].y = lo.y;
          sw[u] = wscl[ke >> 4];
          if (ke + 16 < K) {
            const uint2 hi = *(const uint2 *)(wcodes + (ke >> 1) + 8);
            cw[u].z = hi.x;
            cw[u].w = hi.y;
            sw[u] |= (uint32_t)wscl[(ke >> 4) + 1] << 8;
          }
        }
      }
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
      uint32_t w4[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
      if (L == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = autofp2_codes(w4[i]);
      }
      half8v h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = fp4x8_to_half8(w4[i]);

      if (refine_w) {
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
        if (!row_ok) mb = 0;
        while (mb) {
          const int sg = __ffs(mb) - 1;
          mb &= mb - 1;
          half2v lo, hi;
          offsets_to_half4(woff[pos++], lo, hi);
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
      const _Float16 b0 = (_Float16)e4m3_value(sw[u] & 0xFFu);
      const _Float16 b1 = (_Float16)e4m3_value(sw[u] >> 8);
      h[0] *= b0;
      h[1] *= b0;
      h[2] *= b1;
      h[3] *= b1;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h[i], xv[u][t][i], acc[t], 0, 0, 0);
      }
    }
  }

  // sum the four K quarters
  __shared__ float4v red[4][TT][64];
#pragma unroll
  for (int t = 0; t < TT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
  float scale = (*a.w_T) * (*a.x_T);
  if (L == 2) scale *= a.c2;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float4v s = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
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

}  // namespace

int64_t xh_kpad(int64_t k) { return round_up(k, 128); }

hipError_t launch_act_dequant(const LinearArgs &a, hipStream_t s) {
  const int64_t threads = a.b * (a.kpad / 8);
  hipLaunchKernelGGL(act_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const LinearArgs &a0, hipStream_t s) {
  // slices of at most 64 tokens
  for (int64_t t0 = 0; t0 < a0.b; t0 += 64) {
    LinearArgs a = a0;
    a.b = (a0.b - t0) < 64 ? (a0.b - t0) : 64;
    a.xh = a0.xh + t0 * a0.kpad;
    a.y = (char *)a0.y + t0 * a0.n * (a0.y_dtype == AUTOFP_BF16 ? 2 : 4);
    const dim3 grid((unsigned)((a.n + 15) / 16));
    if (a.b <= 16) {
      hipLaunchKernelGGL((gemv_kernel<1, 8>), grid, dim3(256), 0, s, a);
    } else if (a.b <= 32) {
      hipLaunchKernelGGL((gemv_kernel<2, 4>), grid, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((gemv_kernel<4, 2>), grid, dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace afp
