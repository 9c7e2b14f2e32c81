// AutoFP encode kernels for gfx950: per-tensor scale, NVFP4 base, AutoFP6
// offsets and masks, and the offline weight-mask selection.
//
// "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
// Exponent-Mantissa Refinement" (arXiv 2611.10165v1):
//   App. B.1, Eqs. 2-3   T = amax(X)/(6*448), B_j = E4M3(amax(X_j)/(6T)),
//                        q_i = E2M1(x_i/(T B_j)), round to nearest, ties to even
//   §3.2                 signed offsets d in {-2,-1,0,+1}, delta = d/8,
//                        4-bit subgroup masks, weight mask shared by all rows
//   §6.4, §5.1           activation subgroups refined when NMSE > 0.003,
//                        excluding the weight mask
//   App. E, Alg. 1       weight refinement budget rho*K/4, greedy allocation
//
// Every fp32 step is IEEE-rounded in the order written (no contraction), so
// the codes are a deterministic function of the input.
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_elem(const void *x, int dtype, int64_t i) {
  return dtype == AUTOFP_BF16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// ---------------------------------------------------------------------------
// Producer epilogue ([AE] §6.4: the post-processing unit turns completed
// outputs into the next layer's input activations, non-linear operations
// included): four consecutive elements j .. j + 3 of row r of
//   COPY      v = z[r][j]                         (the first k columns of z)
//   RESIDUAL  v = resid[r][j] + z[r][j]
//   SWIGLU    v = silu(z[r][j]) * z[r][k + j],    silu(g) = g / (1 + e^-g)
// in fp32 (expf, one IEEE division, one product).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float silu_f32(float g) {
#pragma clang fp contract(off)
  return g / (1.0f + expf(-g));
}

__device__ __forceinline__ float4 epilogue4(const EncodeArgs &a, int64_t r, int64_t j) {
#pragma clang fp contract(off)
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

// |v| maxima of the epilogue tensor, one value per block (grid-stride over
// the rows x k/4 quads)
__global__ __launch_bounds__(kThreads) void amax_partial_op_kernel(EncodeArgs a, float *__restrict__ partial) {
  float m = 0.0f;
  const int64_t nq = a.k / 4, tot = a.rows * nq;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < tot; u += (int64_t)gridDim.x * kThreads) {
    const int64_t r = u / nq;
    m = fmaxf(m, max4(epilogue4(a, r, 4 * (u - r * nq))));
  }
  m = wave_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// ---------------------------------------------------------------------------
// Tensor scale: partial maxima, then every encode block folds them (no atomics,
// no zero-initialised scratch, identical T in every block).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const void *__restrict__ x,
                                                                int dtype, int64_t n,
                                                                float *__restrict__ partial) {
  float m = 0.0f;
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < n8; u += stride) {
    if (dtype == AUTOFP_BF16) {
      const uint4 p = ((const uint4 *)x)[u];
      const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = fmaxf(m, fabsf(__uint_as_float(w[j] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
      }
    } else {
      const float4 a = ((const float4 *)x)[2 * u];
      const float4 b = ((const float4 *)x)[2 * u + 1];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    }
  }
  if (blockIdx.x == 0) {
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += kThreads) m = fmaxf(m, fabsf(load_elem(x, dtype, i)));
  }
  m = wave_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// max over the partials, computed by a whole block
__device__ float fold_partials(const float *partial, int n_partial) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n_partial; i += blockDim.x) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  __shared__ float red[16];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Mask prefix (exclusive popcount scan over the packed weight-mask bytes)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void mask_prefix_kernel(const uint8_t *__restrict__ mask,
                                                           int64_t nbytes,
                                                           int32_t *__restrict__ prefix) {
  const int t = threadIdx.x;
  const int64_t per = (nbytes + 1023) / 1024;
  const int64_t b0 = t * per;
  int32_t local = 0;
  for (int64_t i = b0; i < b0 + per && i < nbytes; ++i) local += __popc((uint32_t)mask[i]);
  __shared__ int32_t sc[1024];
  sc[t] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = (t >= off) ? sc[t - off] : 0;
    __syncthreads();
    sc[t] += v;
    __syncthreads();
  }
  int32_t run = sc[t] - local;   // exclusive
  for (int64_t i = b0; i < b0 + per && i < nbytes; ++i) {
    prefix[i] = run;
    run += __popc((uint32_t)mask[i]);
  }
  if (t == 1023) prefix[nbytes] = sc[1023];
}

// ---------------------------------------------------------------------------
// NVFP4 base of two consecutive groups (32 elements), shared by the encoder
// and the weight-gain kernel.
// ---------------------------------------------------------------------------

struct PairEnc {
  float v[32];        // normalized values x / (T B)
  uint32_t q[32];     // E2M1 codes
  uint32_t B[2];      // E4M3 scale codes
};

__device__ __forceinline__ void encode_pair(const float *xv, int ng, float T, float sixT,
                                            PairEnc &e) {
#pragma clang fp contract(off)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g < ng) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xv[16 * g + i]));
      const float b = sixT > 0.0f ? a / sixT : 0.0f;
      const uint32_t B = e4m3_encode(b);
      const float s = T * e4m3_value(B);
      e.B[g] = B;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = (s != 0.0f) ? xv[16 * g + i] / s : 0.0f;
        e.v[16 * g + i] = v;
        e.q[16 * g + i] = e2m1_encode(v);
      }
    } else {
      e.B[g] = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e.v[16 * g + i] = 0.0f;
        e.q[16 * g + i] = 0;
      }
    }
  }
}

__device__ __forceinline__ void load_pair(const void *x, int dtype, int64_t base, int nel,
                                          bool vec_ok, float *xv) {
  if (vec_ok && nel == 32) {
    if (dtype == AUTOFP_BF16) {
      const uint4 *p = (const uint4 *)((const uint16_t *)x + base);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 w = p[c];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xv[8 * c + 2 * j] = __uint_as_float(ww[j] << 16);
          xv[8 * c + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
        }
      }
    } else {
      const float4 *p = (const float4 *)((const float *)x + base);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 w = p[c];
        xv[4 * c] = w.x;
        xv[4 * c + 1] = w.y;
        xv[4 * c + 2] = w.z;
        xv[4 * c + 3] = w.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) xv[i] = (i < nel) ? load_elem(x, dtype, base + i) : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// Encoder: one thread per subgroup (4 elements); the 4 lanes of a quad hold
// one 16-element group and share its amax through DPP quad moves.
// Block (bx, by) covers subgroups [256 bx, 256 bx + 256) of rows by,
// by + gridDim.y, ...
// ---------------------------------------------------------------------------

constexpr int kEncThreads = 256;

__device__ __forceinline__ float quad_max(float v) {
  const float a = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v = fmaxf(v, a);
  const float b = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return fmaxf(v, b);
}

// amax over all n elements, computed by the whole block (small tensors)
__device__ float block_amax_all(const void *x, int dtype, int64_t n) {
  float m = 0.0f;
  const int64_t n8 = n / 8;   // n is a multiple of 16
  for (int64_t u0 = threadIdx.x; u0 < n8; u0 += 4 * kEncThreads) {
    uint4 p[4];
    float4 f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t u = u0 + (int64_t)j * kEncThreads;
      if (dtype == AUTOFP_BF16) {
        p[j] = u < n8 ? ((const uint4 *)x)[u] : make_uint4(0, 0, 0, 0);
      } else {
        f[2 * j] = u < n8 ? ((const float4 *)x)[2 * u] : make_float4(0.f, 0.f, 0.f, 0.f);
        f[2 * j + 1] = u < n8 ? ((const float4 *)x)[2 * u + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (dtype == AUTOFP_BF16) {
        const uint32_t w[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
          m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
        }
      } else {
        const float4 a = f[2 * j], b = f[2 * j + 1];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
        m = fmaxf(m, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
      }
    }
  }
  m = wave_max(m);
  __shared__ float red[kEncThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kEncThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

// amax of the whole epilogue tensor, computed by the block (small tensors)
__device__ float block_amax_op(const EncodeArgs &a) {
  float m = 0.0f;
  const int64_t nq = a.k / 4, tot = a.rows * nq;
  for (int64_t u = threadIdx.x; u < tot; u += kEncThreads) {
    const int64_t r = u / nq;
    m = fmaxf(m, max4(epilogue4(a, r, 4 * (u - r * nq))));
  }
  m = wave_max(m);
  __shared__ float red[kEncThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kEncThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <bool SMALL>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(EncodeArgs a) {
#pragma clang fp contract(off)
  const float amax = SMALL ? (a.op ? block_amax_op(a) : block_amax_all(a.x, a.dtype, a.rows * a.k))
                           : fold_partials(a.partial, a.n_partial);
  const float T = amax / 2688.0f;
  const float sixT = 6.0f * T;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.tensor_scale = T;

  const int64_t ns = a.k / 4;                                  // subgroups per row
  const int64_t mb = (a.k + 31) / 32;                          // mask bytes per row
  const int64_t s = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
  const bool live = s < ns;
  const int lane = threadIdx.x & 63;
  const bool want_act = a.act_refine != 0;
  const bool want_w = a.w_mask != nullptr;
  const uint32_t ex = (want_act && a.exclude_mask && live) ? ((uint32_t)a.exclude_mask[s >> 3] >> (s & 7)) & 1u : 0u;
  uint32_t wbyte = 0;
  int32_t wpos = 0;
  if (want_w && live) {
    wbyte = a.w_mask[s >> 3];
    wpos = a.w_prefix[s >> 3] + __popc(wbyte & ((1u << (s & 7)) - 1u));
  }

  for (int64_t row = blockIdx.y; row < a.rows; row += gridDim.y) {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (live && a.op) {
      const float4 v4 = epilogue4(a, row, 4 * s);
      x[0] = v4.x;
      x[1] = v4.y;
      x[2] = v4.z;
      x[3] = v4.w;
      if (a.v_out) *(float4 *)(a.v_out + row * a.k + 4 * s) = v4;
    } else if (live) {
      const int64_t e = row * a.k + 4 * s;
      if (a.dtype == AUTOFP_BF16) {
        const uint2 p = *(const uint2 *)((const uint16_t *)a.x + e);
        x[0] = __uint_as_float(p.x << 16);
        x[1] = __uint_as_float(p.x & 0xFFFF0000u);
        x[2] = __uint_as_float(p.y << 16);
        x[3] = __uint_as_float(p.y & 0xFFFF0000u);
      } else {
        const float4 p = *(const float4 *)((const float *)a.x + e);
        x[0] = p.x;
        x[1] = p.y;
        x[2] = p.z;
        x[3] = p.w;
      }
    }
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
    if (!want_act && !want_w) continue;

    // offsets d = argmin |r - d/8|, r = v - q (exact in fp32)
    uint32_t ob = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) ob |= offset_code(v[i] - e2m1_value(q[i])) << (2 * i);

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
        a.act_offsets[row * ns + s] = (uint8_t)(refine ? ob : 0u);
        if ((s & 7) == 0) a.act_mask[row * mb + (s >> 3)] = (uint8_t)(bits >> lane);
      }
    }
    // the mask's popcount should equal n_refined; a mask with more refined
    // subgroups writes only the first n_refined of each row
    if (want_w && live && ((wbyte >> (s & 7)) & 1u) && wpos < a.n_refined)
      a.w_offsets[row * (int64_t)a.n_refined + wpos] = (uint8_t)ob;
  }
}

// ---------------------------------------------------------------------------
// Weight-mask selection ([AE] App. E, Alg. 1 allocation, identity Hessian)
// ---------------------------------------------------------------------------

// Per row and subgroup: g = sum_e (eb^2 - er^2) in fp64, eb = w - TB q,
// er = w - TB (q + d/8), TB = T * B exactly.
__global__ __launch_bounds__(kThreads) void weight_gain_kernel(const float *__restrict__ w,
                                                               int64_t rows, int64_t k,
                                                               const float *partial, int n_partial,
                                                               double *__restrict__ row_gain) {
#pragma clang fp contract(off)
  const float amax = fold_partials(partial, n_partial);
  const float T = amax / 2688.0f;
  const float sixT = 6.0f * T;
  const int64_t P2 = (k + 31) / 32;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * P2) return;
  const int64_t row = idx / P2;
  const int64_t pr = idx - row * P2;
  const int64_t k0 = pr * 32;
  const int nel = (int)((k - k0) < 32 ? (k - k0) : 32);
  float xv[32];
  load_pair(w, AUTOFP_F32, row * k + k0, nel, (k % 32) == 0, xv);
  PairEnc e;
  encode_pair(xv, nel / 16, T, sixT, e);
  double *dst = row_gain + row * (k / 4) + k0 / 4;
#pragma unroll
  for (int sg = 0; sg < 8; ++sg) {
    if (sg >= nel / 4) break;
    const double tb = (double)T * (double)e4m3_value(e.B[sg >> 2]);
    double g = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int el = 4 * sg + i;
      const double q = (double)e2m1_value(e.q[el]);
      const uint32_t dc = offset_code(e.v[el] - e2m1_value(e.q[el]));
      const double d = (double)((int)dc - (int)((dc & 2u) << 1));
      const double x = (double)xv[el];
      const double eb = x - tb * q;
      const double er = x - tb * (q + d / 8.0);
      const double ge = eb * eb - er * er;
      g = (i == 0) ? ge : g + ge;
    }
    dst[sg] = g;
  }
}

// Column sums over rows in row order (fp64).
__global__ __launch_bounds__(kThreads) void gain_colsum_kernel(const double *__restrict__ row_gain,
                                                               int64_t rows, int64_t ncol,
                                                               double *__restrict__ col_gain) {
#pragma clang fp contract(off)
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= ncol) return;
  double acc = 0.0;
  for (int64_t n = 0; n < rows; ++n) acc = acc + row_gain[n * ncol + c];
  col_gain[c] = acc;
}

// The two best subgroups of each group (gain descending, then subgroup).
__global__ __launch_bounds__(kThreads) void gain_candidates_kernel(const double *__restrict__ col_gain,
                                                                   int64_t ngroups,
                                                                   double *__restrict__ cgain,
                                                                   int32_t *__restrict__ csg) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= ngroups) return;
  double g[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) g[s] = col_gain[4 * j + s];
  int best = 0;
  for (int s = 1; s < 4; ++s)
    if (g[s] > g[best]) best = s;
  int second = best == 0 ? 1 : 0;
  for (int s = 0; s < 4; ++s)
    if (s != best && g[s] > g[second]) second = s;
  // equal gains rank the lower subgroup first
  for (int s = 0; s < 4; ++s)
    if (s != best && g[s] == g[second] && s < second) second = s;
  cgain[2 * j] = g[best];
  csg[2 * j] = best;
  cgain[2 * j + 1] = g[second];
  csg[2 * j + 1] = second;
}

// rank(c) = number of candidates ordered before c by (gain desc, group, subgroup);
// selected iff rank < budget.
__global__ __launch_bounds__(kThreads) void gain_rank_kernel(const double *__restrict__ cgain,
                                                             const int32_t *__restrict__ csg,
                                                             int64_t ncand, int32_t budget,
                                                             int32_t *__restrict__ selected) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool live = c < ncand;
  const double gc = live ? cgain[c] : 0.0;
  const int64_t jc = c >> 1;
  const int32_t sc = live ? csg[c] : 0;
  __shared__ double tg[kThreads];
  __shared__ int32_t ts[kThreads];
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < ncand; t0 += kThreads) {
    const int64_t t = t0 + threadIdx.x;
    tg[threadIdx.x] = t < ncand ? cgain[t] : 0.0;
    ts[threadIdx.x] = t < ncand ? csg[t] : 0;
    __syncthreads();
    const int64_t lim = (ncand - t0) < kThreads ? (ncand - t0) : kThreads;
    for (int64_t i = 0; i < lim; ++i) {
      const double g = tg[i];
      const int64_t j = (t0 + i) >> 1;
      const int32_t s = ts[i];
      const bool before = (g > gc) || (g == gc && (j < jc || (j == jc && s < sc)));
      rank += before ? 1 : 0;
    }
    __syncthreads();
  }
  if (live) selected[c] = rank < budget ? 1 : 0;
}

__global__ __launch_bounds__(kThreads) void mask_write_kernel(const int32_t *__restrict__ csg,
                                                              const int32_t *__restrict__ selected,
                                                              int64_t ngroups,
                                                              uint8_t *__restrict__ mask) {
  const int64_t pb = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // mask byte
  if (pb >= (ngroups + 1) / 2) return;
  uint32_t byte = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t j = 2 * pb + h;
    if (j >= ngroups) break;
    uint32_t nib = 0;
    for (int c = 0; c < 2; ++c)
      if (selected[2 * j + c]) nib |= 1u << csg[2 * j + c];
    byte |= nib << (4 * h);
  }
  mask[pb] = (uint8_t)byte;
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

int amax_partial_count(int64_t n) {
  const int64_t per_block = (int64_t)kThreads * 8 * 4;
  int64_t b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > kAmaxBlocks) b = kAmaxBlocks;
  return (int)b;
}

hipError_t launch_amax_partial(const void *x, int dtype, int64_t n, float *partial, int n_partial,
                               hipStream_t s) {
  hipLaunchKernelGGL(amax_partial_kernel, dim3(n_partial), dim3(kThreads), 0, s, x, dtype, n, partial);
  return hipGetLastError();
}

hipError_t launch_amax_partial_op(const EncodeArgs &a, float *partial, int n_partial, hipStream_t s) {
  hipLaunchKernelGGL(amax_partial_op_kernel, dim3(n_partial), dim3(kThreads), 0, s, a, partial);
  return hipGetLastError();
}

hipError_t launch_mask_prefix(const uint8_t *mask, int64_t nbytes, int32_t *prefix, hipStream_t s) {
  hipLaunchKernelGGL(mask_prefix_kernel, dim3(1), dim3(1024), 0, s, mask, nbytes, prefix);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, bool small, hipStream_t s) {
  const int64_t ns = a.k / 4;
  const int64_t gx = (ns + kEncThreads - 1) / kEncThreads;
  // rows per block: enough blocks to fill the chip, few enough that the
  // per-block amax fold stays small next to the encode work
  int64_t gy = (16384 + gx - 1) / gx;
  gy = gy < a.rows ? gy : a.rows;
  gy = gy < 65535 ? gy : 65535;
  const dim3 grid((unsigned)gx, (unsigned)gy);
  if (small) hipLaunchKernelGGL(encode_kernel<true>, grid, dim3(kEncThreads), 0, s, a);
  else hipLaunchKernelGGL(encode_kernel<false>, grid, dim3(kEncThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_mask(const float *w, int64_t rows, int64_t k, int32_t budget,
                              const float *partial, int n_partial, double *row_gain,
                              double *col_gain, uint8_t *mask_out, hipStream_t s) {
  const int64_t P2 = (k + 31) / 32;
  const int64_t ncol = k / 4;
  const int64_t ngroups = k / 16;
  double *cgain = col_gain + ncol;
  int32_t *csg = (int32_t *)(cgain + 2 * ngroups);
  int32_t *sel = csg + 2 * ngroups;
  hipLaunchKernelGGL(weight_gain_kernel, dim3(grid_for(rows * P2, kThreads)), dim3(kThreads), 0, s,
                     w, rows, k, partial, n_partial, row_gain);
  hipLaunchKernelGGL(gain_colsum_kernel, dim3(grid_for(ncol, kThreads)), dim3(kThreads), 0, s,
                     row_gain, rows, ncol, col_gain);
  hipLaunchKernelGGL(gain_candidates_kernel, dim3(grid_for(ngroups, kThreads)), dim3(kThreads), 0, s,
                     col_gain, ngroups, cgain, csg);
  hipLaunchKernelGGL(gain_rank_kernel, dim3(grid_for(2 * ngroups, kThreads)), dim3(kThreads), 0, s,
                     cgain, csg, 2 * ngroups, budget, sel);
  hipLaunchKernelGGL(mask_write_kernel, dim3(grid_for((ngroups + 1) / 2, kThreads)), dim3(kThreads),
                     0, s, csg, sel, ngroups, mask_out);
  return hipGetLastError();
}

}  // namespace afp
