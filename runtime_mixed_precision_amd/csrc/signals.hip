// Runtime-policy signals for gfx950 ("AutoEMatic", arXiv 2611.10165v1, §3.1):
//   G_E  normalized Shannon entropy of the top-K next-token logits (K = 10)
//   L_A  ||H_l - H_(l-1)||_2 / (||H_(l-1)||_2 + eps)             (Eq. 1)
// Both are single-pass reductions, one block per row.
#include <hip/hip_runtime.h>
#include <math.h>

#include "afp_device.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kEntThreads = 512;

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

template <int KM>
__global__ __launch_bounds__(kEntThreads) void entropy_topk_kernel(const float *__restrict__ logits,
                                                                   int64_t vocab, int top_k,
                                                                   float *__restrict__ out) {
  const float *z = logits + (int64_t)blockIdx.x * vocab;
  float lst[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) lst[j] = -INFINITY;
  const bool vec = (vocab & 3) == 0;
  if (vec) {
    const float4 *z4 = (const float4 *)z;
    for (int64_t i = threadIdx.x; i < vocab / 4; i += kEntThreads) {
      const float4 v = z4[i];
      if (v.x > lst[KM - 1]) topk_insert(lst, v.x);
      if (v.y > lst[KM - 1]) topk_insert(lst, v.y);
      if (v.z > lst[KM - 1]) topk_insert(lst, v.z);
      if (v.w > lst[KM - 1]) topk_insert(lst, v.w);
    }
  } else {
    for (int64_t i = threadIdx.x; i < vocab; i += kEntThreads) {
      const float v = z[i];
      if (v > lst[KM - 1]) topk_insert(lst, v);
    }
  }
  // merge the per-thread sorted lists: top_k rounds of a block-wide max of the heads
  __shared__ float wbest[kEntThreads / 64];
  __shared__ int wowner[kEntThreads / 64];
  __shared__ float picked[32];
  int head = 0;
  for (int r = 0; r < top_k; ++r) {
    float h = -INFINITY;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j == head) h = lst[j];
    float best = h;
    int owner = threadIdx.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oo = __shfl_xor(owner, o, 64);
      if (ob > best || (ob == best && oo < owner)) {
        best = ob;
        owner = oo;
      }
    }
    if ((threadIdx.x & 63) == 0) {
      wbest[threadIdx.x >> 6] = best;
      wowner[threadIdx.x >> 6] = owner;
    }
    __syncthreads();
    float gb = wbest[0];
    int go = wowner[0];
    for (int w = 1; w < kEntThreads / 64; ++w) {
      if (wbest[w] > gb || (wbest[w] == gb && wowner[w] < go)) {
        gb = wbest[w];
        go = wowner[w];
      }
    }
    if ((int)threadIdx.x == go) ++head;
    if (threadIdx.x == 0) picked[r] = gb;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double m = (double)picked[0];
    double s = 0.0, s1 = 0.0;
    for (int r = 0; r < top_k; ++r) {
      const double t = (double)picked[r] - m;
      const double e = exp(t);
      s += e;
      s1 += t * e;
    }
    const double h = log(s) - s1 / s;
    out[blockIdx.x] = top_k > 1 ? (float)(h / log((double)top_k)) : 0.0f;
  }
}

// Whole-vocabulary entropy with an online log-sum-exp: per thread
// (m, S = sum e^(z-m), S1 = sum (z-m) e^(z-m)); H = ln S - S1 / S.
__global__ __launch_bounds__(kEntThreads) void entropy_full_kernel(const float *__restrict__ logits,
                                                                   int64_t vocab,
                                                                   float *__restrict__ out) {
  const float *z = logits + (int64_t)blockIdx.x * vocab;
  double m = -INFINITY, s = 0.0, s1 = 0.0;
  for (int64_t i = threadIdx.x; i < vocab; i += kEntThreads) {
    const double v = (double)z[i];
    if (v > m) {
      const double sc = (m == -INFINITY) ? 0.0 : exp(m - v);
      s1 = (m == -INFINITY) ? 0.0 : sc * (s1 + (m - v) * s);
      s = sc * s + 1.0;
      m = v;
    } else {
      const double t = v - m;
      const double e = exp(t);
      s += e;
      s1 += t * e;
    }
  }
  __shared__ double sm[kEntThreads], ss[kEntThreads], ss1[kEntThreads];
  sm[threadIdx.x] = m;
  ss[threadIdx.x] = s;
  ss1[threadIdx.x] = s1;
  __syncthreads();
  for (int half = kEntThreads / 2; half > 0; half >>= 1) {
    if ((int)threadIdx.x < half) {
      const double ma = sm[threadIdx.x], mb = sm[threadIdx.x + half];
      const double sa = ss[threadIdx.x], sb = ss[threadIdx.x + half];
      const double s1a = ss1[threadIdx.x], s1b = ss1[threadIdx.x + half];
      const double mm = fmax(ma, mb);
      double rs = 0.0, rs1 = 0.0;
      if (ma != -INFINITY) {
        const double ea = exp(ma - mm);
        rs += ea * sa;
        rs1 += ea * (s1a + (ma - mm) * sa);
      }
      if (mb != -INFINITY) {
        const double eb = exp(mb - mm);
        rs += eb * sb;
        rs1 += eb * (s1b + (mb - mm) * sb);
      }
      sm[threadIdx.x] = mm;
      ss[threadIdx.x] = rs;
      ss1[threadIdx.x] = rs1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double h = log(ss[0]) - ss1[0] / ss[0];
    out[blockIdx.x] = vocab > 1 ? (float)(h / log((double)vocab)) : 0.0f;
  }
}

__device__ __forceinline__ float load_h(const void *p, int dtype, int64_t i) {
  return dtype == AUTOFP_BF16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

__global__ __launch_bounds__(256) void update_norm_kernel(const void *__restrict__ hp,
                                                          const void *__restrict__ hc, int dtype,
                                                          int64_t hidden, float eps,
                                                          float *__restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * hidden;
  double num = 0.0, den = 0.0;
  for (int64_t i = threadIdx.x; i < hidden; i += 256) {
    const float p = load_h(hp, dtype, base + i);
    const float c = load_h(hc, dtype, base + i);
    const double d = (double)c - (double)p;
    num += d * d;
    den += (double)p * (double)p;
  }
  num = wave_sum_d(num);
  den = wave_sum_d(den);
  __shared__ double rn[4], rd[4];
  if ((threadIdx.x & 63) == 0) {
    rn[threadIdx.x >> 6] = num;
    rd[threadIdx.x >> 6] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double n = rn[0] + rn[1] + rn[2] + rn[3];
    const double d = rd[0] + rd[1] + rd[2] + rd[3];
    out[blockIdx.x] = (float)(sqrt(n) / (sqrt(d) + (double)eps));
  }
}

// ---------------------------------------------------------------------------
// Runtime precision policy ([AE] §3.1, Table 1), one thread per sequence.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void trend(autofp_policy_state &s, double m) {
  if (m > s.mean) {
    s.up += 1;
    s.down = 0;
  } else if (m < s.mean) {
    s.down += 1;
    s.up = 0;
  } else {
    s.up = 0;
    s.down = 0;
  }
}

__global__ __launch_bounds__(256) void policy_update_kernel(PolicyArgs a) {
#pragma clang fp contract(off)
  int mx = 0;
  for (int64_t b = threadIdx.x; b < a.batch; b += 256) {
    autofp_policy_state s = a.state[b];
    if (a.layer == 0) {
      if (a.new_sequence) {
        s.mean = 0.0;
        s.m2 = 0.0;
        s.count = 0;
      }
      s.up = 0;
      s.down = 0;
      s.spike = 0;
      s.bits = a.phase == 0 ? 6 : 4;
    }
    const double la = (double)a.l_a[b];
    int p = s.bits;
    double m;
    if (a.phase == 0) {
      m = la;
      if (!s.spike) {
        if (s.count >= 2 && m > s.mean + 3.0 * sqrt(s.m2 / (double)s.count)) s.spike = 1;
      } else {
        trend(s, m);
        if (s.up >= a.n_p) {
          p = p + 2 > 6 ? 6 : p + 2;
          s.up = 0;
        } else if (s.down >= a.n_p) {
          p = p - 2 < 2 ? 2 : p - 2;
          s.down = 0;
        }
      }
    } else {
      const double g = (double)a.g_e[b];
      m = a.lambda_d * la + (1.0 - a.lambda_d) * g;
      const bool high = g >= a.tau;
      const int n_up = high ? a.beta : a.alpha;
      const int n_down = high ? a.alpha : a.beta;
      if (s.count) {
        trend(s, m);
        if (s.up >= n_up) {
          p = p + 2 > 6 ? 6 : p + 2;
          s.up = 0;
        } else if (s.down >= n_down) {
          p = p - 2 < 2 ? 2 : p - 2;
          s.down = 0;
        }
      }
    }
    s.count += 1;
    const double delta = m - s.mean;
    s.mean += delta / (double)s.count;
    s.m2 += delta * (m - s.mean);
    s.bits = p;
    a.state[b] = s;
    a.bits_rows[b] = p;
    mx = p > mx ? p : mx;
  }
  if (a.bits_layer) {
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
      for (int w = 1; w < 4; ++w) r = red[w] > r ? red[w] : r;
      *a.bits_layer = r;
    }
  }
}

}  // namespace

hipError_t launch_policy_update(const PolicyArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(policy_update_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_entropy(const float *logits, int64_t batch, int64_t vocab, int top_k, float *out,
                          hipStream_t s) {
  if (top_k >= vocab) {
    hipLaunchKernelGGL(entropy_full_kernel, dim3((unsigned)batch), dim3(kEntThreads), 0, s, logits,
                       vocab, out);
  } else if (top_k <= 10) {
    hipLaunchKernelGGL(entropy_topk_kernel<10>, dim3((unsigned)batch), dim3(kEntThreads), 0, s,
                       logits, vocab, top_k, out);
  } else {
    hipLaunchKernelGGL(entropy_topk_kernel<32>, dim3((unsigned)batch), dim3(kEntThreads), 0, s,
                       logits, vocab, top_k, out);
  }
  return hipGetLastError();
}

hipError_t launch_update_norm(const void *h_prev, const void *h_cur, int dtype, int64_t batch,
                              int64_t hidden, float eps, float *out, hipStream_t s) {
  hipLaunchKernelGGL(update_norm_kernel, dim3((unsigned)batch), dim3(256), 0, s, h_prev, h_cur, dtype,
                     hidden, eps, out);
  return hipGetLastError();
}

}  // namespace afp
