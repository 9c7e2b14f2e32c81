// Runtime-policy signals for gfx950 ("AutoEMatic", arXiv 2611.10165v1, §3.1):
//   G_E  normalized Shannon entropy of the top-K next-token logits (K = 10)
//   L_A  ||H_l - H_(l-1)||_2 / (||H_(l-1)||_2 + eps)             (Eq. 1)
// G_E reads the logits once (slices of the vocabulary in parallel, then a
// merge of the per-slice candidates); L_A is one block per row.
#include <hip/hip_runtime.h>
#include <math.h>

#include "afp_device.h"
#include "afp_launch.h"
#include "afp_policy.h"

namespace afp {

namespace {

constexpr int kEntThreads = 256;                 // 4 wavefronts
constexpr int kEntPer = 16;                      // logits per thread in the slice pass
constexpr int kEntSlice = kEntThreads * kEntPer; // logits per block in the slice pass
constexpr int kEntWaves = kEntThreads / 64;

// Insert v into a descending list of KM values (the smallest drops out).
template <int KM>
__device__ __forceinline__ void topk_insert(float (&lst)[KM], float v) {
  float cur = v;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const float hi = fmaxf(lst[j], cur);
    cur = fminf(lst[j], cur);
    lst[j] = hi;
  }
}

// Top `top_k` values of the union of the 64 lanes' descending lists: round r
// takes the largest list head (DPP max, lowest lane on ties) and pops it. Lane
// r of the result holds the r-th largest value (-inf for r >= top_k).
template <int KM>
__device__ __forceinline__ float wave_topk(const float (&lst)[KM], int top_k) {
  const int lane = threadIdx.x & 63;
  int head = 0;
  float mine = -INFINITY;
  for (int r = 0; r < top_k; ++r) {
    float h = -INFINITY;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j == head) h = lst[j];
    const uint32_t hu = f32_order(h);
    const uint32_t best = wave_max_u32(hu);
    const uint64_t who = __ballot(hu == best);
    const int owner = __ffsll((unsigned long long)who) - 1;
    if (lane == owner) ++head;
    if (lane == r) mine = f32_unorder(best);
  }
  return mine;
}

// Top `top_k` values of a block's per-thread lists, in lanes 0 .. top_k - 1 of
// wavefront 0 (other lanes and wavefronts: -inf).
template <int KM>
__device__ __forceinline__ float block_topk(const float (&lst)[KM], int top_k) {
  __shared__ float wtop[kEntWaves * KM];
  const int lane = threadIdx.x & 63;
  const float t = wave_topk(lst, top_k);
  if (lane < top_k) wtop[(threadIdx.x >> 6) * top_k + lane] = t;
  __syncthreads();
  float l2[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) l2[j] = -INFINITY;
  if (threadIdx.x < 64)
    for (int i = lane; i < kEntWaves * top_k; i += 64) topk_insert(l2, wtop[i]);
  return threadIdx.x < 64 ? wave_topk(l2, top_k) : -INFINITY;
}

// Slice pass: block (s, row) reads logits [s * kEntSlice, (s + 1) * kEntSlice)
// of its row once and writes its top_k values to cand[row][s][0 .. top_k).
template <int KM>
__global__ __launch_bounds__(kEntThreads) void entropy_slice_kernel(const float *__restrict__ logits,
                                                                    int64_t vocab, int top_k,
                                                                    float *__restrict__ cand) {
  const int64_t row = blockIdx.y;
  const float *z = logits + row * vocab;
  const int64_t base = (int64_t)blockIdx.x * kEntSlice;
  float v[kEntPer];
  if ((vocab & 3) == 0) {
    // 4 x 16-byte loads per thread, all issued before any is used
#pragma unroll
    for (int j = 0; j < kEntPer / 4; ++j) {
      const int64_t i = base + 4 * (threadIdx.x + (int64_t)j * kEntThreads);
      float4 q = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (i < vocab) q = *(const float4 *)(z + i);
      v[4 * j] = q.x;
      v[4 * j + 1] = q.y;
      v[4 * j + 2] = q.z;
      v[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kEntPer; ++j) {
      const int64_t i = base + threadIdx.x + (int64_t)j * kEntThreads;
      v[j] = i < vocab ? z[i] : -INFINITY;
    }
  }
  float lst[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) lst[j] = -INFINITY;
#pragma unroll
  for (int j = 0; j < kEntPer; ++j) topk_insert(lst, v[j]);
  const float t = block_topk(lst, top_k);
  if (threadIdx.x < (unsigned)top_k) cand[(row * gridDim.x + blockIdx.x) * top_k + threadIdx.x] = t;
}

// Merge pass: one wavefront per row over its n_cand candidates, then
// G_E = (ln S - S1 / S) / ln(top_k) with S = sum e^(z - m), S1 = sum (z - m) e^(z - m)
// over the top_k values (m the largest), in fp64.
template <int KM>
__global__ __launch_bounds__(64) void entropy_merge_kernel(const float *__restrict__ cand,
                                                           int64_t n_cand, int top_k,
                                                           float *__restrict__ out) {
  const float *c = cand + (int64_t)blockIdx.x * n_cand;
  const int lane = threadIdx.x;
  float lst[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) lst[j] = -INFINITY;
  for (int64_t i0 = lane; i0 < n_cand; i0 += 8 * 64) {
    float v[8];   // eight independent loads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (i0 + 64 * u < n_cand) ? c[i0 + 64 * u] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) topk_insert(lst, v[u]);
  }
  const float f = wave_topk(lst, top_k);
  const double m = (double)__shfl(f, 0, 64);
  double e = 0.0, te = 0.0;
  // a candidate of -inf (fewer than top_k finite logits) has probability 0
  // and adds nothing to S or S1
  if (lane < top_k && f != -INFINITY) {
    const double d = (double)f - m;
    e = exp(d);
    te = d * e;
  }
  const double S = wave_sum_d(e);
  const double S1 = wave_sum_d(te);
  if (lane == 0) out[blockIdx.x] = top_k > 1 ? (float)((log(S) - S1 / S) / log((double)top_k)) : 0.0f;
}

// Whole-vocabulary entropy, slice pass: per block (m, S, S1) with
// S = sum e^(z - m), S1 = sum (z - m) e^(z - m) over its slice (fp64).
struct LseAcc {
  double m, s, s1;
};

__device__ __forceinline__ LseAcc lse_merge(LseAcc a, LseAcc b) {
  if (a.m == -INFINITY) return b;
  if (b.m == -INFINITY) return a;
  const double mm = fmax(a.m, b.m);
  const double ea = exp(a.m - mm), eb = exp(b.m - mm);
  LseAcc r;
  r.m = mm;
  r.s = ea * a.s + eb * b.s;
  r.s1 = ea * (a.s1 + (a.m - mm) * a.s) + eb * (b.s1 + (b.m - mm) * b.s);
  return r;
}

__device__ __forceinline__ LseAcc wave_lse(LseAcc a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    LseAcc b;
    b.m = __shfl_xor(a.m, o, 64);
    b.s = __shfl_xor(a.s, o, 64);
    b.s1 = __shfl_xor(a.s1, o, 64);
    a = lse_merge(a, b);
  }
  return a;
}

__device__ LseAcc block_lse(LseAcc a) {
  __shared__ double sm[kEntWaves][3];
  a = wave_lse(a);
  if ((threadIdx.x & 63) == 0) {
    sm[threadIdx.x >> 6][0] = a.m;
    sm[threadIdx.x >> 6][1] = a.s;
    sm[threadIdx.x >> 6][2] = a.s1;
  }
  __syncthreads();
  LseAcc r{-INFINITY, 0.0, 0.0};
  for (int w = 0; w < kEntWaves; ++w) r = lse_merge(r, LseAcc{sm[w][0], sm[w][1], sm[w][2]});
  return r;
}

__global__ __launch_bounds__(kEntThreads) void entropy_full_slice_kernel(const float *__restrict__ logits,
                                                                         int64_t vocab,
                                                                         double *__restrict__ part) {
  const int64_t row = blockIdx.y;
  const float *z = logits + row * vocab;
  const int64_t base = (int64_t)blockIdx.x * kEntSlice;
  float v[kEntPer];
#pragma unroll
  for (int j = 0; j < kEntPer; ++j) {
    const int64_t i = base + threadIdx.x + (int64_t)j * kEntThreads;
    v[j] = i < vocab ? z[i] : -INFINITY;
  }
  double m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kEntPer; ++j) m = fmax(m, (double)v[j]);
  LseAcc a{m, 0.0, 0.0};
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kEntPer; ++j) {
      if (v[j] != -INFINITY) {
        const double t = (double)v[j] - m;
        const double e = exp(t);
        a.s += e;
        a.s1 += t * e;
      }
    }
  }
  a = block_lse(a);
  if (threadIdx.x == 0) {
    double *p = part + 3 * (row * gridDim.x + blockIdx.x);
    p[0] = a.m;
    p[1] = a.s;
    p[2] = a.s1;
  }
}

__global__ __launch_bounds__(kEntThreads) void entropy_full_merge_kernel(const double *__restrict__ part,
                                                                         int64_t n_part, int64_t vocab,
                                                                         float *__restrict__ out) {
  const double *p = part + 3 * (int64_t)blockIdx.x * n_part;
  LseAcc a{-INFINITY, 0.0, 0.0};
  for (int64_t i = threadIdx.x; i < n_part; i += kEntThreads)
    a = lse_merge(a, LseAcc{p[3 * i], p[3 * i + 1], p[3 * i + 2]});
  a = block_lse(a);
  if (threadIdx.x == 0) out[blockIdx.x] = vocab > 1 ? (float)((log(a.s) - a.s1 / a.s) / log((double)vocab)) : 0.0f;
}

__device__ __forceinline__ float load_h(const void *p, int dtype, int64_t i) {
  return dtype == AUTOFP_BF16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

// 8 consecutive hidden-state values as fp32 (16- or 32-byte aligned vector loads)
__device__ __forceinline__ void load8_h(const void *p, int dtype, int64_t i8, float (&v)[8]) {
  if (dtype == AUTOFP_BF16) {
    const uint4 q = ((const uint4 *)p)[i8];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4 a = ((const float4 *)p)[2 * i8];
    const float4 b = ((const float4 *)p)[2 * i8 + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

constexpr int kNormThreads = 256;
constexpr int kNormUnroll = 4;   // vectors of 8 per thread loaded before any is used
// Rows up to which policy_layer_kernel computes L_A itself. It takes the rows
// one after another: at 16 rows the 32-layer step took 5.6 ms against 4.6 ms
// with the separate L_A launch.
constexpr int kPolicyLayerFusedRows = 4;

// L_A of one row ([AE] Eq. 1) by a block of kNormThreads threads: fp64 sums of
// (h_cur - h_prev)^2 and h_prev^2 in a fixed partition (thread, then
// wavefront, then the block in wavefront order), so every kernel that calls it
// gets the same value. The result is valid in thread 0.
__device__ float row_update_norm(const void *__restrict__ hp, const void *__restrict__ hc, int dtype,
                                 int64_t hidden, int64_t base, float eps, double *rn, double *rd) {
  double num = 0.0, den = 0.0;
  if ((hidden & 7) == 0 && (((uintptr_t)hp | (uintptr_t)hc) & 15) == 0) {
    const int64_t n8 = hidden / 8, b8 = base / 8;
    for (int64_t i0 = threadIdx.x; i0 < n8; i0 += kNormUnroll * kNormThreads) {
      float p[kNormUnroll][8], c[kNormUnroll][8];
#pragma unroll
      for (int u = 0; u < kNormUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * kNormThreads;
        if (i < n8) {
          load8_h(hp, dtype, b8 + i, p[u]);
          load8_h(hc, dtype, b8 + i, c[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) p[u][j] = c[u][j] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < kNormUnroll; ++u) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double d = (double)c[u][j] - (double)p[u][j];
          num += d * d;
          den += (double)p[u][j] * (double)p[u][j];
        }
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < hidden; i += kNormThreads) {
      const float p = load_h(hp, dtype, base + i);
      const float c = load_h(hc, dtype, base + i);
      const double d = (double)c - (double)p;
      num += d * d;
      den += (double)p * (double)p;
    }
  }
  num = wave_sum_d(num);
  den = wave_sum_d(den);
  if ((threadIdx.x & 63) == 0) {
    rn[threadIdx.x >> 6] = num;
    rd[threadIdx.x >> 6] = den;
  }
  __syncthreads();
  float out = 0.0f;
  if (threadIdx.x == 0) {
    double n = 0.0, d = 0.0;
    for (int w = 0; w < kNormThreads / 64; ++w) {
      n += rn[w];
      d += rd[w];
    }
    out = (float)(sqrt(n) / (sqrt(d) + (double)eps));
  }
  __syncthreads();   // rn / rd may be reused by the next row
  return out;
}

__global__ __launch_bounds__(kNormThreads) void update_norm_kernel(const void *__restrict__ hp,
                                                                   const void *__restrict__ hc, int dtype,
                                                                   int64_t hidden, float eps,
                                                                   float *__restrict__ out) {
  __shared__ double rn[kNormThreads / 64], rd[kNormThreads / 64];
  const float v = row_update_norm(hp, hc, dtype, hidden, (int64_t)blockIdx.x * hidden, eps, rn, rd);
  if (threadIdx.x == 0) out[blockIdx.x] = v;
}

// ---------------------------------------------------------------------------
// Runtime precision policy ([AE] §3.1, Table 1), one thread per sequence
// (the step itself: policy_row, afp_policy.h).
// ---------------------------------------------------------------------------

// highest level over the block's threads' rows -> *bits_layer
__device__ void write_layer_max(int mx, int32_t *bits_layer) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int v = __shfl_xor(mx, o, 64);
    mx = v > mx ? v : mx;
  }
  __shared__ int red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    int r = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = red[w] > r ? red[w] : r;
    *bits_layer = r;
  }
}

__global__ __launch_bounds__(256) void policy_update_kernel(PolicyArgs a) {
  int mx = 0;
  for (int64_t b = threadIdx.x; b < a.batch; b += 256) {
    const int p = policy_row(a, b, (double)a.l_a[b]);
    mx = p > mx ? p : mx;
  }
  if (a.bits_layer) write_layer_max(mx, a.bits_layer);
}

// L_A of every row (the same partition as update_norm_kernel) and the policy
// step, in one block: for a few rows one launch instead of two.
__global__ __launch_bounds__(kNormThreads) void policy_layer_kernel(PolicyArgs a) {
  __shared__ double rn[kNormThreads / 64], rd[kNormThreads / 64];
  int mx = 0;
  for (int64_t b = 0; b < a.batch; ++b) {
    const float la = row_update_norm(a.h_prev, a.h_cur, a.h_dtype, a.hidden, b * a.hidden, a.eps, rn, rd);
    if (threadIdx.x == 0) {
      a.l_a_out[b] = la;
      const int p = policy_row(a, b, (double)la);
      mx = p > mx ? p : mx;
    }
  }
  if (a.bits_layer) write_layer_max(mx, a.bits_layer);
}

}  // namespace

hipError_t launch_policy_update(const PolicyArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(policy_update_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_policy_layer(const PolicyArgs &a, hipStream_t s) {
  if (a.batch <= kPolicyLayerFusedRows) {
    hipLaunchKernelGGL(policy_layer_kernel, dim3(1), dim3(kNormThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(update_norm_kernel, dim3((unsigned)a.batch), dim3(kNormThreads), 0, s, a.h_prev, a.h_cur,
                     a.h_dtype, a.hidden, a.eps, a.l_a_out);
  PolicyArgs b = a;
  b.l_a = a.l_a_out;
  hipLaunchKernelGGL(policy_update_kernel, dim3(1), dim3(256), 0, s, b);
  return hipGetLastError();
}

int64_t entropy_slices(int64_t vocab) { return (vocab + kEntSlice - 1) / kEntSlice; }

size_t entropy_workspace_bytes(int64_t batch, int64_t vocab) {
  const size_t topk = (size_t)batch * (size_t)entropy_slices(vocab) * 32 * sizeof(float);
  const size_t full = (size_t)batch * (size_t)entropy_slices(vocab) * 3 * sizeof(double);
  return topk > full ? topk : full;
}

hipError_t launch_entropy(const float *logits, int64_t batch, int64_t vocab, int top_k, float *out,
                          void *ws, hipStream_t s) {
  const int64_t ns = entropy_slices(vocab);
  const dim3 grid((unsigned)ns, (unsigned)batch);
  if (top_k >= vocab) {
    hipLaunchKernelGGL(entropy_full_slice_kernel, grid, dim3(kEntThreads), 0, s, logits, vocab,
                       (double *)ws);
    hipLaunchKernelGGL(entropy_full_merge_kernel, dim3((unsigned)batch), dim3(kEntThreads), 0, s,
                       (const double *)ws, ns, vocab, out);
  } else if (top_k <= 10) {
    hipLaunchKernelGGL(entropy_slice_kernel<10>, grid, dim3(kEntThreads), 0, s, logits, vocab, top_k,
                       (float *)ws);
    hipLaunchKernelGGL(entropy_merge_kernel<10>, dim3((unsigned)batch), dim3(64), 0, s,
                       (const float *)ws, ns * top_k, top_k, out);
  } else {
    hipLaunchKernelGGL(entropy_slice_kernel<32>, grid, dim3(kEntThreads), 0, s, logits, vocab, top_k,
                       (float *)ws);
    hipLaunchKernelGGL(entropy_merge_kernel<32>, dim3((unsigned)batch), dim3(64), 0, s,
                       (const float *)ws, ns * top_k, top_k, out);
  }
  return hipGetLastError();
}

hipError_t launch_update_norm(const void *h_prev, const void *h_cur, int dtype, int64_t batch,
                              int64_t hidden, float eps, float *out, hipStream_t s) {
  hipLaunchKernelGGL(update_norm_kernel, dim3((unsigned)batch), dim3(kNormThreads), 0, s, h_prev, h_cur, dtype,
                     hidden, eps, out);
  return hipGetLastError();
}

}  // namespace afp
