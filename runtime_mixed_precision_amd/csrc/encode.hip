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
#include "afp_encode.h"
#include "afp_policy.h"
#include "afp_launch.h"

namespace afp {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_elem(const void *x, int dtype, int64_t i) {
  return dtype == AUTOFP_BF16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
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

// RESIDUAL_RMSNORM row scales: block r sums the squares of u = resid + z of
// row r in fp64 (each square exact; thread t takes quads t, t + 256, ...,
// then the wavefronts' butterfly sums and the four wavefront sums in order:
// one fixed order) and writes c = 1 / sqrt(sum / k + eps) rounded to fp32.
__global__ __launch_bounds__(kThreads) void rowscale_kernel(EncodeArgs a) {
#pragma clang fp contract(off)
  const int64_t r = blockIdx.x;
  double acc = 0.0;
  for (int64_t q = threadIdx.x; q < a.k / 4; q += kThreads) {
    const float4 u = resid_sum4(a, r, 4 * q);
    acc += (double)u.x * (double)u.x;
    acc += (double)u.y * (double)u.y;
    acc += (double)u.z * (double)u.z;
    acc += (double)u.w * (double)u.w;
  }
  acc = wave_sum_d_dpp(acc);
  __shared__ double red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = red[0];
    for (int w = 1; w < kThreads / 64; ++w) t += red[w];
    a.rowscale[r] = (float)(1.0 / sqrt(t / (double)a.k + kRmsEps));
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
// Encoders: one thread per subgroup (4 elements); the 4 lanes of a quad hold
// one 16-element group and share its amax through DPP quad moves.
// ---------------------------------------------------------------------------

constexpr int kEncThreads = 256;

// Encoder of larger tensors: T from the amax partials of the previous launch;
// block (bx, by) covers subgroups [256 bx, 256 bx + 256) of rows by,
// by + gridDim.y, ...
__global__ __launch_bounds__(kEncThreads) void encode_kernel(EncodeArgs a) {
  const float T = tensor_scale_of(a, fold_partials(a.partial, a.n_partial));
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.tensor_scale = T;
  const int64_t ns = a.k / 4;
  const int64_t s = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
  const bool live = s < ns;
  const bool fp6g = a.fmt == AUTOFP_FMT_FP6G;
  const uint32_t ex = (a.act_refine && a.exclude_mask && live) ? ((uint32_t)a.exclude_mask[s >> 3] >> (s & 7)) & 1u : 0u;
  uint32_t wbyte = 0;
  int32_t wpos = 0;
  if (a.w_mask && live) {
    wbyte = a.w_mask[s >> 3];
    wpos = a.w_prefix[s >> 3] + __popc(wbyte & ((1u << (s & 7)) - 1u));
  }
  for (int64_t row = blockIdx.y; row < a.rows; row += gridDim.y) {
    float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
      if (a.op == AUTOFP_EPI_RESIDUAL_RMSNORM) {
        const float4 u4 = resid_sum4(a, row, 4 * s);
        v4 = scale4(u4, a.rowscale[row]);
        if (a.v_out) *(float4 *)(a.v_out + row * a.k + 4 * s) = u4;   // the hidden state
      } else {
        v4 = load_quad(a, row, s);
        if (a.op && a.v_out) *(float4 *)(a.v_out + row * a.k + 4 * s) = v4;
      }
    }
    if (fp6g) encode_subgroup_fp6g(a, T, row, s, live, v4);
    else encode_subgroup(a, T, row, s, live, v4, ex, wbyte, wpos);
  }
}

// ---------------------------------------------------------------------------
// One-launch encoder of small tensors (rows * roundup(k/4, 64) <= 8192
// subgroup slots): slot u holds subgroup s = u mod nqp of row u / nqp, nqp =
// k/4 rounded up to 64 (so a wavefront never spans two rows). Block bx of TPB
// threads encodes slots [TPB bx, TPB bx + TPB); every block loads all slots
// (thread t: slots j TPB + t, j < SPT, SPT the block count rounded up to a
// power of two), takes the amax of the whole tensor from them and encodes
// its own slot from the registers: one round trip to memory, no second
// launch. 256 threads a block up to 4096 slots (one wavefront per SIMD: the
// per-slot encode is a chain of dependent instructions), 512 above and for
// SwiGLU (every block reads the whole tensor, so fewer, larger blocks). The source is fixed at compile time and
// every load of a thread (its slots' inputs, then the mask bytes the encode
// needs) is issued before the first use of any, so the loads of a thread
// overlap instead of waiting one after another.
// ---------------------------------------------------------------------------
constexpr int kSmallSlots = 8192;
constexpr int kSmallSlots256 = 4096;   // up to here 256-thread blocks, above 512

// The raw inputs of the four elements of subgroup s of row `row`: p = x (SRC
// 0 fp32, 1 bf16) or z (the epilogue ops, SRC = 1 + op; 6: RESIDUAL_RMSNORM
// with the layer's policy step); q = the residual (residual ops) or the up
// half z[k + j] (SwiGLU). Loads only.
template <int SRC>
__device__ __forceinline__ void src_load(const EncodeArgs &a, int32_t row, int32_t s, float4 &p, float4 &q) {
  if constexpr (SRC == 0) {
    p = *(const float4 *)((const float *)a.x + (int64_t)row * a.k + 4 * s);
  } else if constexpr (SRC == 1) {
    const uint2 v = *(const uint2 *)((const uint16_t *)a.x + (int64_t)row * a.k + 4 * s);
    p = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                    __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
  } else {
    p = *(const float4 *)(a.z + (int64_t)row * a.ldz + 4 * s);
    if constexpr (SRC == 1 + AUTOFP_EPI_RESIDUAL || SRC >= 1 + AUTOFP_EPI_RESIDUAL_RMSNORM)
      q = *(const float4 *)(a.resid + (int64_t)row * a.k + 4 * s);
    else if constexpr (SRC == 1 + AUTOFP_EPI_SWIGLU)
      q = *(const float4 *)(a.z + (int64_t)row * a.ldz + a.k + 4 * s);
  }
}

// The tensor value from the raw inputs (epilogue4's arithmetic, the op fixed
// at compile time): x or z; resid + z; silu(z) * up; RESIDUAL_RMSNORM: the
// residual sum u (the row scale applies later).
template <int SRC>
__device__ __forceinline__ float4 src_value(float4 p, float4 q) {
#pragma clang fp contract(off)
  if constexpr (SRC == 1 + AUTOFP_EPI_RESIDUAL || SRC >= 1 + AUTOFP_EPI_RESIDUAL_RMSNORM) {
    return make_float4(q.x + p.x, q.y + p.y, q.z + p.z, q.w + p.w);
  } else if constexpr (SRC == 1 + AUTOFP_EPI_SWIGLU) {
    return make_float4(silu_f32(p.x) * q.x, silu_f32(p.y) * q.y, silu_f32(p.z) * q.z, silu_f32(p.w) * q.w);
  } else {
    return p;
  }
}

// The layer's policy step beside the RESIDUAL_RMSNORM encode (one extra block
// of the launch): the new hidden state u = resid + z (the same fp32 sums the
// encode blocks write to v_out), per 64-slot chunk the fp64 sums of
// (u - h_prev)^2 and h_prev^2 (Eq. 1; differences and squares exact in fp64,
// lane order fixed by the butterfly), per row the chunks in order, L_A, then
// the Table 1 step of every row in order with the highest level to
// bits_layer.
template <int TPB, int SPT>
__device__ __forceinline__ void policy_tail(const EncodeArgs &a, int32_t nqp) {
  __shared__ double cnum[kSmallSlots / 64], cden[kSmallSlots / 64];
  __shared__ float la_s[kSmallSlots / 64];
  const int32_t nq = (int32_t)(a.k / 4);
  const int32_t tot = (int32_t)a.rows * nqp;
  const float inv_nqp = 1.0f / (float)nqp;
  float4 z[SPT], rr[SPT], hp[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int32_t uj = j * TPB + (int32_t)threadIdx.x;
    const int32_t r = (int32_t)(((float)uj + 0.5f) * inv_nqp), sq = uj - r * nqp;
    const bool ok = uj < tot && sq < nq;
    const int64_t e = (int64_t)(ok ? r : 0) * a.k + 4 * (ok ? sq : 0);
    z[j] = *(const float4 *)(a.z + (int64_t)(ok ? r : 0) * a.ldz + 4 * (ok ? sq : 0));
    rr[j] = *(const float4 *)(a.resid + e);
    hp[j] = *(const float4 *)((const float *)a.pol.h_prev + e);
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
#pragma clang fp contract(off)
    const int32_t uj = j * TPB + (int32_t)threadIdx.x;
    const int32_t r = (int32_t)(((float)uj + 0.5f) * inv_nqp), sq = uj - r * nqp;
    const bool ok = uj < tot && sq < nq;
    const float c[4] = {rr[j].x + z[j].x, rr[j].y + z[j].y, rr[j].z + z[j].z, rr[j].w + z[j].w};
    const float pv[4] = {hp[j].x, hp[j].y, hp[j].z, hp[j].w};
    double nm = 0.0, dn = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double df = ok ? (double)c[e] - (double)pv[e] : 0.0;
      const double pd = ok ? (double)pv[e] : 0.0;
      nm += df * df;
      dn += pd * pd;
    }
    nm = wave_sum_d_dpp(nm);
    dn = wave_sum_d_dpp(dn);
    if ((threadIdx.x & 63) == 0 && uj < tot) {
      cnum[uj / 64] = nm;
      cden[uj / 64] = dn;
    }
  }
  __syncthreads();
  const int32_t cpr = nqp / 64;
  if ((int32_t)threadIdx.x < (int32_t)a.rows) {
    double n = 0.0, d = 0.0;
    for (int32_t c = 0; c < cpr; ++c) {
      n += cnum[(int32_t)threadIdx.x * cpr + c];
      d += cden[(int32_t)threadIdx.x * cpr + c];
    }
    const float la = (float)(sqrt(n) / (sqrt(d) + (double)a.pol.eps));
    la_s[threadIdx.x] = la;
    a.pol.l_a_out[threadIdx.x] = la;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int mx = 0;
    for (int64_t b = 0; b < a.rows; ++b) {
      const int lv = policy_row(a.pol, b, (double)la_s[b]);
      mx = lv > mx ? lv : mx;
    }
    if (a.pol.bits_layer) *a.pol.bits_layer = mx;
  }
}

template <int TPB, int SPT, int SRC>
__global__ __launch_bounds__(TPB) void encode_small_kernel(EncodeArgs a, int32_t nqp) {
  static_assert((SPT & (SPT - 1)) == 0 && TPB * SPT <= kSmallSlots, "slot groups per thread: a power of two");
  constexpr bool NORM = SRC >= 1 + AUTOFP_EPI_RESIDUAL_RMSNORM;
  constexpr bool POL = SRC == 2 + AUTOFP_EPI_RESIDUAL_RMSNORM;   // with the policy step
  const int32_t nq = (int32_t)(a.k / 4);
  const int32_t tot = (int32_t)a.rows * nqp;
  const int bx = (int)blockIdx.x;
  const int32_t u = bx * TPB + (int32_t)threadIdx.x;
  const int32_t row = u / nqp, s = u - row * nqp;
  const bool live = u < tot && s < nq;
  const bool fp6g = a.fmt == AUTOFP_FMT_FP6G;
  if constexpr (POL) {
    // the last block runs the layer's policy step beside the encode blocks
    if (bx == (int)gridDim.x - 1) {
      policy_tail<TPB, SPT>(a, nqp);
      return;
    }
  }
  // row of slot uj without an integer division: (uj + 1/2) / nqp lies at
  // least 1/(2 nqp) inside its integer interval, and the fp32 product errs by
  // at most (rows + 1) 2^-23 (uj < (rows + 1) nqp), below 2^-8 of that margin
  // since rows nqp <= 8192
  const float inv_nqp = 1.0f / (float)nqp;
  auto row_of = [&](int32_t uj) { return (int32_t)(((float)uj + 0.5f) * inv_nqp); };
  // slot groups in the order bx, bx + 1, ... (mod SPT): the first is the
  // block's own; an absent slot reads slot 0 and counts as zero
  float4 p[SPT], q[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int32_t uj = ((bx + j) & (SPT - 1)) * TPB + (int32_t)threadIdx.x;
    const int32_t r = row_of(uj), sq = uj - r * nqp;
    const bool ok = uj < tot && sq < nq;
    src_load<SRC>(a, ok ? r : 0, ok ? sq : 0, p[j], q[j]);
  }
  // mask bytes of the own slot (read at slot 0 when absent, unused then)
  const int32_t sl = live ? s : 0;
  uint32_t exb = 0, wb = 0;
  int32_t wp = 0;
  if (!fp6g && a.act_refine && a.exclude_mask) exb = a.exclude_mask[sl >> 3];
  if (!fp6g && a.w_mask) {
    wb = a.w_mask[sl >> 3];
    wp = a.w_prefix[sl >> 3];
  }
  float m = 0.0f;
  float4 own = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 own_u = own;   // RESIDUAL_RMSNORM: the residual sum of the own slot
  if constexpr (NORM) {
    // u of every slot; per 64-slot chunk (one row: nqp is a multiple of 64)
    // the fp64 sum of the exact squares, lane order fixed by the butterfly;
    // then per row the chunk sums in order and c = 1 / sqrt(sum / k + eps)
    __shared__ double chunk[kSmallSlots / 64];
    __shared__ float rsc[kSmallSlots / 64];   // at most 64 rows: nqp >= 64
    float4 uu[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = ((bx + j) & (SPT - 1)) * TPB + (int32_t)threadIdx.x;
      const int32_t r = row_of(uj), sq = uj - r * nqp;
      const bool ok = uj < tot && sq < nq;
      uu[j] = ok ? src_value<SRC>(p[j], q[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
      double d = (double)uu[j].x * (double)uu[j].x;
      d += (double)uu[j].y * (double)uu[j].y;
      d += (double)uu[j].z * (double)uu[j].z;
      d += (double)uu[j].w * (double)uu[j].w;
      d = wave_sum_d_dpp(d);
      if ((threadIdx.x & 63) == 0 && uj < tot) chunk[uj / 64] = d;
    }
    __syncthreads();
    const int32_t cpr = nqp / 64;   // chunks per row
    if ((int32_t)threadIdx.x < (int32_t)a.rows) {
      double t = 0.0;
      for (int32_t c = 0; c < cpr; ++c) t += chunk[(int32_t)threadIdx.x * cpr + c];
      rsc[threadIdx.x] = (float)(1.0 / sqrt(t / (double)a.k + kRmsEps));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = ((bx + j) & (SPT - 1)) * TPB + (int32_t)threadIdx.x;
      const int32_t r = row_of(uj);
      const float4 v = uj < tot ? scale4(uu[j], rsc[r]) : make_float4(0.f, 0.f, 0.f, 0.f);
      m = fmaxf(m, max4(v));
      if (j == 0) {
        own = v;
        own_u = uu[0];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = ((bx + j) & (SPT - 1)) * TPB + (int32_t)threadIdx.x;
      const int32_t r = row_of(uj), sq = uj - r * nqp;
      const bool ok = uj < tot && sq < nq;
      const float4 v = ok ? src_value<SRC>(p[j], q[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
      m = fmaxf(m, max4(v));
      if (j == 0) own = v;
    }
  }
  m = wave_max(m);
  __shared__ float red[TPB / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int w = 1; w < TPB / 64; ++w) amax = fmaxf(amax, red[w]);
  const float T = tensor_scale_of(a, amax);
  if (bx == 0 && threadIdx.x == 0) *a.tensor_scale = T;

  if (SRC >= 2 && live && a.v_out)
    *(float4 *)(a.v_out + (int64_t)row * a.k + 4 * s) = NORM ? own_u : own;
  if (fp6g) {
    encode_subgroup_fp6g(a, T, row, s, live, own);
  } else {
    const uint32_t ex = (a.act_refine && a.exclude_mask && live) ? (exb >> (s & 7)) & 1u : 0u;
    const int32_t wpos = wp + __popc(wb & ((1u << (s & 7)) - 1u));
    encode_subgroup(a, T, row, s, live, own, ex, live ? wb : 0u, live ? wpos : 0);
  }
}

// ---------------------------------------------------------------------------
// Element-parallel one-launch encoder (AutoFP6 activations; every source but
// SwiGLU): one thread per element instead of per four-element subgroup, so
// each thread's encode is about a quarter of the work. The decisions a
// subgroup or group shares come from DPP moves among its lanes (lanes 16g ..
// 16g + 15 hold group g of a wavefront, four lanes a subgroup): the group
// maximum, the subgroup's NMSE sums in element order, its offset byte and the
// code byte of an element pair. Every block still loads every slot of the
// tensor for the maximum (and the RMSNorm row sums); the own element is one
// more load. Rows are padded to 4 nqp elements (a multiple of 256), so a
// wavefront (64 consecutive elements of one row) holds 4 whole groups.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// The raw inputs of element `col` of row `row` (src_load for one element).
template <int SRC>
__device__ __forceinline__ void src_load1(const EncodeArgs &a, int32_t row, int32_t col, float &p, float &q) {
  if constexpr (SRC == 0) {
    p = ((const float *)a.x)[(int64_t)row * a.k + col];
  } else if constexpr (SRC == 1) {
    p = __uint_as_float((uint32_t)((const uint16_t *)a.x)[(int64_t)row * a.k + col] << 16);
  } else {
    p = a.z[(int64_t)row * a.ldz + col];
    if constexpr (SRC == 1 + AUTOFP_EPI_RESIDUAL || SRC >= 1 + AUTOFP_EPI_RESIDUAL_RMSNORM)
      q = a.resid[(int64_t)row * a.k + col];
  }
}

// encode_subgroup's arithmetic for the AutoFP6 format, one element per lane
// (the same values and bytes): E2M1 code and E4M3 group scale; with
// act_refine the subgroup's offsets and its refinement decision outside the
// exclusion mask (exb: the mask byte of the lane's subgroup).
__device__ __forceinline__ void encode_element(const EncodeArgs &a, float T, int32_t row, int32_t col, bool live,
                                               float x, uint32_t exb) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int32_t k = (int32_t)a.k;
  const float sixT = 6.0f * T;
  // the group's maximum: quads, then the half rows and rows of 16 lanes
  float gm = fabsf(x);
  gm = fmaxf(gm, dppf<0xB1>(gm));
  gm = fmaxf(gm, dppf<0x4E>(gm));
  gm = fmaxf(gm, dppf<0x141>(gm));
  gm = fmaxf(gm, dppf<0x140>(gm));
  const float b = sixT > 0.0f ? gm / sixT : 0.0f;
  const uint32_t B = e4m3_encode(b);
  const float sc = T * e4m3_value(B);
  const float v = (sc != 0.0f) ? x / sc : 0.0f;
  const uint32_t q = e2m1_encode(v);
  const uint32_t qn = dppu<0xF5>(q);   // the odd neighbour's code (quad lanes 1, 1, 3, 3)
  if (live && !(col & 1)) a.codes[(int64_t)row * (k / 2) + (col >> 1)] = (uint8_t)(q | (qn << 4));
  if (live && !(col & 15)) a.scales[(int64_t)row * (k / 16) + (col >> 4)] = (uint8_t)B;
  if (!a.act_refine) return;
  const float r = v - e2m1_value(q);
  const uint32_t oc = offset_code(r);
  const float rr = r * r;
  const float vv = v * v;
  // the subgroup's sums in element order, ((e0 + e1) + e2) + e3, in all 4 lanes
  const float num = ((dppf<0x00>(rr) + dppf<0x55>(rr)) + dppf<0xAA>(rr)) + dppf<0xFF>(rr);
  const float den = ((dppf<0x00>(vv) + dppf<0x55>(vv)) + dppf<0xAA>(vv)) + dppf<0xFF>(vv);
  const uint32_t ob = dppu<0x00>(oc) | (dppu<0x55>(oc) << 2) | (dppu<0xAA>(oc) << 4) | (dppu<0xFF>(oc) << 6);
  const uint32_t s = (uint32_t)col >> 2;
  const bool ex = a.exclude_mask != nullptr && ((exb >> (s & 7)) & 1u);
  const bool refine = live && den > 0.0f && num > a.thresh * den && !ex;
  const uint64_t bits = __ballot(refine);
  if (live && !(col & 3)) a.act_offsets[(int64_t)row * (k / 4) + s] = (uint8_t)(refine ? ob : 0u);
  if (live && !(col & 31)) {
    // 8 subgroups' bits (every fourth lane of the lane's half wavefront) -> one mask byte
    uint32_t w = (uint32_t)(bits >> (lane & 32)) & 0x11111111u;
    w = (w | (w >> 3)) & 0x03030303u;
    w = (w | (w >> 6)) & 0x000F000Fu;
    w = (w | (w >> 12)) & 0xFFu;
    a.act_mask[(int64_t)row * ((k + 31) / 32) + (s >> 3)] = (uint8_t)w;
  }
}

template <int TPB, int SPT, int SRC>
__global__ __launch_bounds__(TPB) void encode_elem_kernel(EncodeArgs a, int32_t nqp) {
  static_assert((SPT & (SPT - 1)) == 0 && TPB * SPT <= kSmallSlots, "slot groups per thread: a power of two");
  static_assert(SRC != 1 + AUTOFP_EPI_SWIGLU, "SwiGLU keeps the per-subgroup kernel");
  constexpr bool NORM = SRC >= 1 + AUTOFP_EPI_RESIDUAL_RMSNORM;
  constexpr bool POL = SRC == 2 + AUTOFP_EPI_RESIDUAL_RMSNORM;
  const int bx = (int)blockIdx.x;
  if constexpr (POL) {
    if (bx == (int)gridDim.x - 1) {
      policy_tail<TPB, SPT>(a, nqp);
      return;
    }
  }
  const int32_t nq = (int32_t)(a.k / 4);
  const int32_t tot = (int32_t)a.rows * nqp;
  const int32_t kp = 4 * nqp;
  // rows without integer division: (u + 1/2) / d lies at least 1/(2 d) inside
  // its integer interval, and the fp32 product errs by at most (rows + 2)
  // 2^-23 (u < (rows + 2) d), below a fortieth of that margin since
  // rows 4 nqp <= 32768 and 4 nqp <= 32768
  const float inv_nqp = 1.0f / (float)nqp;
  auto row_of = [&](int32_t uj) { return (int32_t)(((float)uj + 0.5f) * inv_nqp); };
  const int32_t e = bx * TPB + (int32_t)threadIdx.x;
  const int32_t erow = (int32_t)(((float)e + 0.5f) * (0.25f * inv_nqp));
  const int32_t ecol = e - erow * kp;
  const bool live = erow < a.rows && ecol < a.k;
  // every load first: the own element, every slot, the own subgroup's mask byte
  float op = 0.0f, oq = 0.0f;
  src_load1<SRC>(a, live ? erow : 0, live ? ecol : 0, op, oq);
  float4 p[SPT], q[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int32_t uj = j * TPB + (int32_t)threadIdx.x;
    const int32_t r = row_of(uj), sq = uj - r * nqp;
    const bool ok = uj < tot && sq < nq;
    src_load<SRC>(a, ok ? r : 0, ok ? sq : 0, p[j], q[j]);
  }
  uint32_t exb = 0;
  if (a.act_refine && a.exclude_mask) exb = a.exclude_mask[(live ? ecol : 0) >> 5];

  float m = 0.0f;
  float rs = 1.0f;   // RESIDUAL_RMSNORM: the own row's scale
  if constexpr (NORM) {
    __shared__ double chunk[kSmallSlots / 64];
    __shared__ float rsc[kSmallSlots / 64];
    float4 uu[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = j * TPB + (int32_t)threadIdx.x;
      const int32_t r = row_of(uj), sq = uj - r * nqp;
      const bool ok = uj < tot && sq < nq;
      uu[j] = ok ? src_value<SRC>(p[j], q[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
      double d = (double)uu[j].x * (double)uu[j].x;
      d += (double)uu[j].y * (double)uu[j].y;
      d += (double)uu[j].z * (double)uu[j].z;
      d += (double)uu[j].w * (double)uu[j].w;
      d = wave_sum_d_dpp(d);
      if ((threadIdx.x & 63) == 0 && uj < tot) chunk[uj / 64] = d;
    }
    __syncthreads();
    const int32_t cpr = nqp / 64;
    if ((int32_t)threadIdx.x < (int32_t)a.rows) {
      double t = 0.0;
      for (int32_t c = 0; c < cpr; ++c) t += chunk[(int32_t)threadIdx.x * cpr + c];
      rsc[threadIdx.x] = (float)(1.0 / sqrt(t / (double)a.k + kRmsEps));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = j * TPB + (int32_t)threadIdx.x;
      const float4 v = uj < tot ? scale4(uu[j], rsc[row_of(uj)]) : make_float4(0.f, 0.f, 0.f, 0.f);
      m = fmaxf(m, max4(v));
    }
    rs = rsc[live ? erow : 0];
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int32_t uj = j * TPB + (int32_t)threadIdx.x;
      const int32_t r = row_of(uj), sq = uj - r * nqp;
      const bool ok = uj < tot && sq < nq;
      const float4 v = ok ? src_value<SRC>(p[j], q[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
      m = fmaxf(m, max4(v));
    }
  }
  m = wave_max(m);
  __shared__ float red[TPB / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int w = 1; w < TPB / 64; ++w) amax = fmaxf(amax, red[w]);
  const float T = tensor_scale_of(a, amax);
  if (bx == 0 && threadIdx.x == 0) *a.tensor_scale = T;

  // the own element: v (RESIDUAL_RMSNORM: u times the row scale)
  float u1, x;
  {
#pragma clang fp contract(off)
    u1 = (SRC == 1 + AUTOFP_EPI_RESIDUAL || NORM) ? oq + op : op;
    x = NORM ? u1 * rs : u1;
  }
  x = live ? x : 0.0f;
  if (SRC >= 2 && live && a.v_out) a.v_out[(int64_t)erow * a.k + ecol] = u1;
  encode_element(a, T, erow, ecol, live, x, exb);
}

}  // namespace

int64_t encode_slots_per_row(int64_t k) { return (k / 4 + 63) / 64 * 64; }

bool encode_is_small(int64_t rows, int64_t k) {
  return rows >= 1 && rows * encode_slots_per_row(k) <= kSmallSlots;
}

namespace {

// ---------------------------------------------------------------------------
// Weight-mask selection ([AE] App. E, Alg. 1 allocation, identity Hessian)
// ---------------------------------------------------------------------------

// Per row and subgroup: g = sum_e (eb^2 - er^2) in fp64, eb = w - TB q,
// er = w - TB (q + d/8), TB = T * B exactly.
__global__ __launch_bounds__(kThreads) void weight_gain_kernel(const float *__restrict__ w,
                                                               int64_t rows, int64_t k,
                                                               const float *partial, int n_partial,
                                                               double *__restrict__ row_gain, int fmt,
                                                               const double *__restrict__ hdiag) {
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
      const float r = e.v[el] - e2m1_value(e.q[el]);
      double delta;
      if (fmt == AUTOFP_FMT_AUTOFP8) {
        delta = (double)offset8(r) / 8.0;
      } else {
        const float inv = fmt == AUTOFP_FMT_AUTOFP6E ? e2m1_inv_pow2e(e.q[el]) : 1.0f;
        const uint32_t dc = offset_code(r * inv);
        delta = (double)((int)dc - (int)((dc & 2u) << 1)) / 8.0 / (double)inv;
      }
      const double x = (double)xv[el];
      const double eb = x - tb * q;
      const double er = x - tb * (q + delta);
      const double ge0 = eb * eb - er * er;
      // Hessian-diagonal weight of the column ([AE] Eq. 7), when given
      const double ge = hdiag ? hdiag[k0 + el] * ge0 : ge0;
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

hipError_t launch_rowscale(const EncodeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(rowscale_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mask_prefix(const uint8_t *mask, int64_t nbytes, int32_t *prefix, hipStream_t s) {
  hipLaunchKernelGGL(mask_prefix_kernel, dim3(1), dim3(1024), 0, s, mask, nbytes, prefix);
  return hipGetLastError();
}

// blocks of TPB threads over rows * nqp slots; SPT = the block count rounded
// up to a power of two
template <int TPB, int SRC>
hipError_t launch_small(const EncodeArgs &a, int32_t nqp, hipStream_t s) {
  const int64_t ge = (a.rows * nqp + TPB - 1) / TPB;   // encode blocks
  int spt = 1;
  while (spt < ge) spt *= 2;
  // with the policy step: one more block, beside the encode blocks
  const int64_t gx = ge + (SRC == 2 + AUTOFP_EPI_RESIDUAL_RMSNORM ? 1 : 0);
#define AFP_SMALL(P)                                                                               \
  case P:                                                                                          \
    if constexpr (TPB * P <= kSmallSlots)                                                          \
      hipLaunchKernelGGL((encode_small_kernel<TPB, P, SRC>), dim3((unsigned)gx), dim3(TPB), 0, s, a, nqp); \
    else                                                                                           \
      return hipErrorInvalidValue;                                                                 \
    break
  switch (spt) {
    AFP_SMALL(1);
    AFP_SMALL(2);
    AFP_SMALL(4);
    AFP_SMALL(8);
    AFP_SMALL(16);
    default: return hipErrorInvalidValue;
  }
#undef AFP_SMALL
  return hipGetLastError();
}

// the element-parallel encoder: rows * 4 nqp elements over blocks of TPB,
// SPT slot groups per thread (the slot count over TPB rounded up to a power of
// two); with the policy step one more block
template <int TPB, int SRC>
hipError_t launch_elem(const EncodeArgs &a, int32_t nqp, hipStream_t s) {
  const int64_t ge = (a.rows * 4 * (int64_t)nqp + TPB - 1) / TPB;
  const int64_t gs = (a.rows * (int64_t)nqp + TPB - 1) / TPB;
  int spt = 1;
  while (spt < gs) spt *= 2;
  const int64_t gx = ge + (SRC == 2 + AUTOFP_EPI_RESIDUAL_RMSNORM ? 1 : 0);
#define AFP_ELEM(P)                                                                                \
  case P:                                                                                          \
    if constexpr (TPB * P <= kSmallSlots)                                                          \
      hipLaunchKernelGGL((encode_elem_kernel<TPB, P, SRC>), dim3((unsigned)gx), dim3(TPB), 0, s, a, nqp); \
    else                                                                                           \
      return hipErrorInvalidValue;                                                                 \
    break
  switch (spt) {
    AFP_ELEM(1);
    AFP_ELEM(2);
    AFP_ELEM(4);
    AFP_ELEM(8);
    AFP_ELEM(16);
    default: return hipErrorInvalidValue;
  }
#undef AFP_ELEM
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s) {
  if (encode_is_small(a.rows, a.k)) {
    const int64_t nqp = encode_slots_per_row(a.k);
    const int src = a.op ? 1 + a.op : (a.dtype == AUTOFP_BF16 ? 1 : 0);
    const int32_t q = (int32_t)nqp;
    const bool big = a.rows * nqp > kSmallSlots256;   // 512-thread blocks
    if (a.fmt == AUTOFP_FMT_AUTOFP6 && a.w_mask == nullptr) {
      // activations: the element-parallel encoder (SwiGLU excepted)
      switch (src) {
        case 0: return big ? launch_elem<512, 0>(a, q, s) : launch_elem<256, 0>(a, q, s);
        case 1: return big ? launch_elem<512, 1>(a, q, s) : launch_elem<256, 1>(a, q, s);
        case 2: return big ? launch_elem<512, 2>(a, q, s) : launch_elem<256, 2>(a, q, s);
        case 3: return big ? launch_elem<512, 3>(a, q, s) : launch_elem<256, 3>(a, q, s);
        case 5:
          if (a.policy) return big ? launch_elem<512, 6>(a, q, s) : launch_elem<256, 6>(a, q, s);
          return big ? launch_elem<512, 5>(a, q, s) : launch_elem<256, 5>(a, q, s);
        default: break;
      }
    }
    switch (src) {
      case 0: return big ? launch_small<512, 0>(a, q, s) : launch_small<256, 0>(a, q, s);
      case 1: return big ? launch_small<512, 1>(a, q, s) : launch_small<256, 1>(a, q, s);
      case 2: return big ? launch_small<512, 2>(a, q, s) : launch_small<256, 2>(a, q, s);
      case 3: return big ? launch_small<512, 3>(a, q, s) : launch_small<256, 3>(a, q, s);
      case 4: return launch_small<512, 4>(a, q, s);
      case 5:
        if (a.policy) return big ? launch_small<512, 6>(a, q, s) : launch_small<256, 6>(a, q, s);
        return big ? launch_small<512, 5>(a, q, s) : launch_small<256, 5>(a, q, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t ns = a.k / 4;
  const int64_t gx = (ns + kEncThreads - 1) / kEncThreads;
  // rows per block: enough blocks to fill the chip, few enough that the
  // per-block amax fold stays small next to the encode work
  int64_t gy = (16384 + gx - 1) / gx;
  gy = gy < a.rows ? gy : a.rows;
  gy = gy < 65535 ? gy : 65535;
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kEncThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_mask(const float *w, int64_t rows, int64_t k, int32_t budget,
                              const float *partial, int n_partial, double *row_gain,
                              double *col_gain, uint8_t *mask_out, int fmt, const double *hdiag,
                              hipStream_t s) {
  const int64_t P2 = (k + 31) / 32;
  const int64_t ncol = k / 4;
  const int64_t ngroups = k / 16;
  double *cgain = col_gain + ncol;
  int32_t *csg = (int32_t *)(cgain + 2 * ngroups);
  int32_t *sel = csg + 2 * ngroups;
  hipLaunchKernelGGL(weight_gain_kernel, dim3(grid_for(rows * P2, kThreads)), dim3(kThreads), 0, s,
                     w, rows, k, partial, n_partial, row_gain, fmt, hdiag);
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
