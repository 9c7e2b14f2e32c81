// Device-side runtime precision policy ([AE] §3.1, Table 1): one step of the
// per-sequence state machine, shared by the policy kernels and the fused tail
// of the layer's last producer epilogue.
//
// "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM Inference via Automatic
// Exponent-Mantissa Refinement" (arXiv 2611.10165v1), §3.1 and Table 1.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "afp_launch.h"

namespace afp {

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

// One policy step for row b with L_A = la (the fp32 value, widened); returns
// the level of the next layer and updates the row's state.
__device__ __forceinline__ int policy_row(const PolicyArgs &a, int64_t b, double la) {
#pragma clang fp contract(off)
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
  return p;
}

}  // namespace afp
