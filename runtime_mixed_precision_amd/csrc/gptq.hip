// Refinement-aware GPTQ calibration for gfx950 ("AutoEMatic", arXiv
// 2611.10165v1, App. E "Refinement-Aware GPTQ Calibration", Algorithm 1 and
// the Hessian-diagonal-weighted group error of Eq. 7).
//
//   T fixed from the original weights (line 4); the refined-subgroup count
//   l_j of every group from the budget allocation on the original weights
//   (lines 5-12: the greedy over marginal reductions of Eq. 7, which is the
//   selection of the budgeted mask with the column gains weighted by H_ii);
//   then for every 16-column group j in order (lines 13-24):
//     encode     B, q, d of each row from the compensated weights (fp64
//                rounded to fp32, the fp32 steps of the encoder)
//     mask       m*_j = the l_j subgroups with the largest Eq. 7 reductions
//                summed over all rows (a tie goes to the lower subgroup)
//     update     codes, scale, offsets of the group; r = W_J - What_J;
//                e U_JJ = r by forward substitution (line 22)
//     propagate  W[:, later] -= e U[J, later] (line 23)
//   The working weights are fp64 in the workspace. Every fp64 product and
//   sum of lines 22-23 is a separate IEEE operation in index order (no fused
//   multiply-add), so the result does not depend on the launch shape.
#include <hip/hip_runtime.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kT = 256;
constexpr int kPropRows = 16;   // rows per propagation block

size_t al(size_t v) { return (v + 255) / 256 * 256; }

struct GptqWs {
  float *partial;
  double *w64, *e, *gpart, *row_gain, *col_gain;
  uint4 *stash;
  uint8_t *amask;
  int32_t *prefix, *msel;
};

size_t select_col_bytes(int64_t k) {
  const size_t ncol = (size_t)(k / 4), ng = (size_t)(k / 16);
  return al(sizeof(double) * (ncol + 2 * ng) + sizeof(int32_t) * 4 * ng);
}

GptqWs carve(void *ws, int64_t rows, int64_t k) {
  char *p = (char *)ws;
  GptqWs g;
  g.partial = (float *)p;
  p += al(sizeof(float) * kAmaxBlocks);
  g.w64 = (double *)p;
  p += al(sizeof(double) * (size_t)rows * (size_t)k);
  g.e = (double *)p;
  p += al(sizeof(double) * (size_t)rows * 16);
  g.gpart = (double *)p;
  p += al(sizeof(double) * (size_t)rows * 4);
  g.stash = (uint4 *)p;
  p += al(sizeof(uint4) * (size_t)rows);
  g.row_gain = (double *)p;
  p += al(sizeof(double) * (size_t)rows * (size_t)(k / 4));
  g.col_gain = (double *)p;
  p += select_col_bytes(k);
  g.amask = (uint8_t *)p;
  p += al((size_t)mask_bytes(k));
  g.prefix = (int32_t *)p;
  p += al(sizeof(int32_t) * (size_t)(mask_bytes(k) + 1));
  g.msel = (int32_t *)p;
  return g;
}

__global__ __launch_bounds__(kT) void gptq_init_kernel(const float *__restrict__ w, int64_t n,
                                                       double *__restrict__ w64) {
  for (int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kT)
    w64[i] = (double)w[i];
}

// T = amax / (6 * 448) from the amax partials (line 4), as the encoder folds them
__global__ __launch_bounds__(kT) void gptq_scale_kernel(const float *__restrict__ partial, int n_partial,
                                                        float *__restrict__ tensor_scale) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n_partial; i += kT) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  __shared__ float red[kT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kT / 64; ++w) r = fmaxf(r, red[w]);
    *tensor_scale = r / 2688.0f;
  }
}

// Lines 15-19 for group j of one row: B, q, d from the compensated weights,
// and the row's Eq. 7 reductions g_s = sum_{i in s} H_ii ((W - TBq)^2 -
// (W - TB(q + d/8))^2) of its four subgroups. stash[n] = (codes of the 16
// elements as nibbles, two words; the four offset bytes; B).
__global__ __launch_bounds__(kT) void gptq_encode_kernel(const double *__restrict__ w64, int64_t rows, int64_t k,
                                                         int64_t j, const float *__restrict__ tensor_scale,
                                                         const double *__restrict__ hdiag,
                                                         double *__restrict__ gpart, uint4 *__restrict__ stash) {
#pragma clang fp contract(off)
  const int64_t n = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (n >= rows) return;
  const float T = *tensor_scale;
  const float sixT = 6.0f * T;
  const double *src = w64 + n * k + 16 * j;
  double W[16];
  float x[16];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    W[i] = src[i];
    x[i] = (float)W[i];
    a = fmaxf(a, fabsf(x[i]));
  }
  const float b = sixT > 0.0f ? a / sixT : 0.0f;
  const uint32_t B = e4m3_encode(b);
  const float sc = T * e4m3_value(B);
  const double tb = (double)T * (double)e4m3_value(B);
  uint32_t qw[2] = {0u, 0u}, dw = 0u;
  double g[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = (sc != 0.0f) ? x[i] / sc : 0.0f;
    const uint32_t q = e2m1_encode(v);
    const uint32_t dc = offset_code(v - e2m1_value(q));
    qw[i >> 3] |= q << (4 * (i & 7));
    dw |= dc << (2 * i);
    const double qv = (double)e2m1_value(q);
    const double dv = (double)((int)dc - (int)((dc & 2u) << 1)) / 8.0;
    const double eb = W[i] - tb * qv;
    const double er = W[i] - tb * (qv + dv);
    const double ge = hdiag[16 * j + i] * (eb * eb - er * er);
    g[i >> 2] = ((i & 3) == 0) ? ge : g[i >> 2] + ge;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) gpart[n * 4 + s] = g[s];
  stash[n] = make_uint4(qw[0], qw[1], dw, B);
}

// Line 20: m*_j = the l_j subgroups (l_j from the allocation mask) with the
// largest reductions summed over the rows; written to msel[j] and to nibble
// j of the output mask (group 2i in the low nibble of byte i).
__global__ __launch_bounds__(kT) void gptq_mask_kernel(const double *__restrict__ gpart, int64_t rows, int64_t j,
                                                       const uint8_t *__restrict__ amask, int32_t *__restrict__ msel,
                                                       uint8_t *__restrict__ mask_out) {
#pragma clang fp contract(off)
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t n = threadIdx.x; n < rows; n += kT) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = acc[s] + gpart[n * 4 + s];
  }
  __shared__ double red[kT / 64][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = wave_sum_d(acc[s]);
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) red[threadIdx.x >> 6][s] = acc[s];
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double G[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    G[s] = red[0][s];
    for (int w = 1; w < kT / 64; ++w) G[s] = G[s] + red[w][s];
  }
  const uint32_t level = __popc(((uint32_t)amask[j >> 1] >> (4 * (j & 1))) & 0xFu);
  uint32_t m = 0;
  for (uint32_t t = 0; t < level && t < 2; ++t) {
    int best = -1;
    for (int s = 0; s < 4; ++s)
      if (!((m >> s) & 1u) && (best < 0 || G[s] > G[best])) best = s;
    m |= 1u << best;
  }
  msel[j] = (int32_t)m;
  if ((j & 1) == 0) mask_out[j >> 1] = (uint8_t)m;
  else mask_out[j >> 1] = (uint8_t)(mask_out[j >> 1] | (m << 4));
}

// Lines 21-22 for group j of one row: the group's codes, scale and offsets
// (compacted: the refined subgroups of row n follow the allocation's order),
// r = W_J - What_J and e with e U_JJ = r.
__global__ __launch_bounds__(kT) void gptq_update_kernel(const double *__restrict__ w64, int64_t rows, int64_t k,
                                                         int64_t j, const float *__restrict__ tensor_scale,
                                                         const double *__restrict__ u, const uint4 *__restrict__ stash,
                                                         const int32_t *__restrict__ msel,
                                                         const uint8_t *__restrict__ amask,
                                                         const int32_t *__restrict__ prefix, int32_t n_refined,
                                                         uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                         uint8_t *__restrict__ offsets, double *__restrict__ e) {
#pragma clang fp contract(off)
  const int64_t n = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (n >= rows) return;
  const uint4 st = stash[n];
  const uint32_t m = (uint32_t)msel[j];
  *(uint2 *)(codes + n * (k / 2) + 8 * j) = make_uint2(st.x, st.y);
  scales[n * (k / 16) + j] = (uint8_t)st.w;
  int32_t pos = prefix[j >> 1] + ((j & 1) ? __popc((uint32_t)amask[j >> 1] & 0xFu) : 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if ((m >> s) & 1u) {
      if (pos < n_refined) offsets[n * (int64_t)n_refined + pos] = (uint8_t)(st.z >> (8 * s));
      ++pos;
    }
  }
  const double tb = (double)(*tensor_scale) * (double)e4m3_value(st.w);
  const double *src = w64 + n * k + 16 * j;
  const double *uj = u + (16 * j) * k + 16 * j;   // U_JJ, row stride k
  double ev[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t q = ((i < 8 ? st.x : st.y) >> (4 * (i & 7))) & 15u;
    const double qv = (double)e2m1_value(q);
    double wh;
    if ((m >> (i >> 2)) & 1u) {
      const uint32_t dc = (st.z >> (2 * i)) & 3u;
      const double dv = (double)((int)dc - (int)((dc & 2u) << 1)) / 8.0;
      wh = tb * (qv + dv);
    } else {
      wh = tb * qv;
    }
    double acc = src[i] - wh;
#pragma unroll
    for (int kk = 0; kk < i; ++kk) acc = acc - ev[kk] * uj[kk * k + i];
    ev[i] = acc / uj[i * k + i];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) e[n * 16 + i] = ev[i];
}

// Line 23: W[n][c] -= sum_i e[n][i] U[16j + i][c] for the later columns c,
// the 16 products accumulated in index order. One thread per column, 16 rows
// per block.
__global__ __launch_bounds__(kT) void gptq_propagate_kernel(double *__restrict__ w64, int64_t rows, int64_t k,
                                                            int64_t j, const double *__restrict__ u,
                                                            const double *__restrict__ e) {
#pragma clang fp contract(off)
  const int64_t c = 16 * (j + 1) + (int64_t)blockIdx.x * kT + threadIdx.x;
  if (c >= k) return;
  double uc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) uc[i] = u[(16 * j + i) * k + c];
  const int64_t r0 = (int64_t)blockIdx.y * kPropRows;
  const int64_t r1 = (r0 + kPropRows) < rows ? (r0 + kPropRows) : rows;
  for (int64_t r = r0; r < r1; ++r) {
    const double *er = e + r * 16;
    double upd = er[0] * uc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) upd = upd + er[i] * uc[i];
    w64[r * k + c] = w64[r * k + c] - upd;
  }
}

inline unsigned blocks_for(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

size_t gptq_workspace_bytes(int64_t rows, int64_t k) {
  return al(sizeof(float) * kAmaxBlocks) + al(sizeof(double) * (size_t)rows * (size_t)k) +
         al(sizeof(double) * (size_t)rows * 16) + al(sizeof(double) * (size_t)rows * 4) +
         al(sizeof(uint4) * (size_t)rows) + al(sizeof(double) * (size_t)rows * (size_t)(k / 4)) +
         select_col_bytes(k) + al((size_t)mask_bytes(k)) + al(sizeof(int32_t) * (size_t)(mask_bytes(k) + 1)) +
         al(sizeof(int32_t) * (size_t)(k / 16));
}

hipError_t launch_gptq(const float *w, int64_t rows, int64_t k, const double *u, const double *hdiag,
                       int32_t budget, const autofp_packed *out, void *ws, hipStream_t s) {
  const GptqWs g = carve(ws, rows, k);
  const int64_t n = rows * k;
  const int np = amax_partial_count(n);
  hipError_t err = launch_amax_partial(w, AUTOFP_F32, n, g.partial, np, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gptq_init_kernel, dim3(blocks_for(n, kT) < 65536u ? blocks_for(n, kT) : 65535u), dim3(kT), 0,
                     s, w, n, g.w64);
  // lines 5-12: the allocation mask (its popcount per group is l_j)
  err = launch_select_mask(w, rows, k, budget, g.partial, np, g.row_gain, g.col_gain, g.amask,
                           AUTOFP_FMT_AUTOFP6, hdiag, s);
  if (err != hipSuccess) return err;
  err = launch_mask_prefix(g.amask, mask_bytes(k), g.prefix, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gptq_scale_kernel, dim3(1), dim3(kT), 0, s, g.partial, np, out->tensor_scale);
  const int64_t G = k / 16;
  const unsigned rb = blocks_for(rows, kT);
  for (int64_t j = 0; j < G; ++j) {
    hipLaunchKernelGGL(gptq_encode_kernel, dim3(rb), dim3(kT), 0, s, g.w64, rows, k, j, out->tensor_scale, hdiag,
                       g.gpart, g.stash);
    hipLaunchKernelGGL(gptq_mask_kernel, dim3(1), dim3(kT), 0, s, g.gpart, rows, j, g.amask, g.msel, out->mask);
    hipLaunchKernelGGL(gptq_update_kernel, dim3(rb), dim3(kT), 0, s, g.w64, rows, k, j, out->tensor_scale, u,
                       g.stash, g.msel, g.amask, g.prefix, out->n_refined, out->codes, out->scales, out->offsets,
                       g.e);
    const int64_t later = k - 16 * (j + 1);
    if (later > 0)
      hipLaunchKernelGGL(gptq_propagate_kernel, dim3(blocks_for(later, kT), blocks_for(rows, kPropRows)), dim3(kT),
                         0, s, g.w64, rows, k, j, u, g.e);
  }
  return hipGetLastError();
}

}  // namespace afp
