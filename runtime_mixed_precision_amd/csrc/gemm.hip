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
// Tiling: a block of 4 wavefronts computes a 128-token x 128-row tile with
// K steps of 64. Each step loads the packed weight tile (16 B of codes and two
// scale bytes per thread, plus refinement offsets at level 6), decodes it into
// LDS, copies the fp16 activation tile into LDS, and each wavefront runs a 2x2
// grid of 32x32x16 MFMAs over its 64x64 quadrant. The next step's global loads
// are issued before the current step's MFMAs.
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

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
            if ((m >> s) & 1u) t.offs[s] = woff[pos++];
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

}  // namespace

hipError_t launch_gemm(const LinearArgs &a, hipStream_t s) {
  const int64_t mtiles = (a.b + BM - 1) / BM;
  const int64_t ntiles = (a.n + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(mtiles * ntiles)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace afp
