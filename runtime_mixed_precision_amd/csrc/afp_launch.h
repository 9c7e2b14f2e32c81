// Host-side launchers shared by the translation units of libautofp (internal;
// the public interface is include/autofp.h). Each returns the hipError_t of
// its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "autofp.h"

namespace afp {

constexpr int kGroup = 16;      // elements per NVFP4 group
constexpr int kAmaxBlocks = 1024;   // max partial-max blocks of the tensor-scale pass

inline int64_t mask_bytes(int64_t k) { return (k + 31) / 32; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// ---- encode.hip ----
// Partial |x| maxima: writes n_partial floats to partial.
hipError_t launch_amax_partial(const void *x, int dtype, int64_t n, float *partial, int n_partial,
                               hipStream_t s);
int amax_partial_count(int64_t n);

// Exclusive prefix of popcounts over the mask bytes: prefix[i] = refined
// subgroups in bytes [0, i); prefix has nbytes + 1 entries.
hipError_t launch_mask_prefix(const uint8_t *mask, int64_t nbytes, int32_t *prefix, hipStream_t s);

// Arguments of the policy step (signals.hip; also the fused tail of the
// RESIDUAL_RMSNORM epilogue in encode.hip).
struct PolicyArgs {
  int phase, layer, new_sequence;
  const float *l_a, *g_e;
  int64_t batch;
  double tau, lambda_d;
  int alpha, beta, n_p;
  autofp_policy_state *state;
  int32_t *bits_rows, *bits_layer;
  // launch_policy_layer: L_A computed from the hidden states into l_a_out
  const void *h_prev, *h_cur;
  int h_dtype;
  int64_t hidden;
  float eps;
  float *l_a_out;
};

struct EncodeArgs {
  const void *x;
  int dtype;
  int64_t rows, k;
  const float *partial;        // amax partials
  int n_partial;
  uint8_t *codes, *scales;
  float *tensor_scale;
  // activation refinement (dense offsets)
  int act_refine;
  const uint8_t *exclude_mask;  // [mask_bytes(k)] or null
  float thresh;
  uint8_t *act_mask;            // [rows][mask_bytes(k)]
  uint8_t *act_offsets;         // [rows][k/4]
  // weight refinement (compacted offsets)
  const uint8_t *w_mask;        // [mask_bytes(k)] or null
  const int32_t *w_prefix;      // mask prefix table
  int32_t n_refined;
  uint8_t *w_offsets;           // [rows][n_refined]
  // element / offset format of the encoded tensor (autofp_format)
  int fmt;
  // producer epilogue (op != 0): the encoded tensor is v = op(z, resid),
  // [rows][k], computed on the fly from z [rows][ldz] fp32 (x is unused) and
  // written to v_out when non-null. Ops: autofp_epilogue_op.
  int op;
  const float *z;
  int64_t ldz;
  const float *resid;           // [rows][k] (residual ops)
  float *v_out;                 // [rows][k] or null (RESIDUAL_RMSNORM: the residual sum u)
  float *rowscale;              // RESIDUAL_RMSNORM, large tensors: the per-row scales c [rows]
  // RESIDUAL_RMSNORM of small tensors with policy != 0: the layer's policy
  // step in the same launch (L_A of each row from pol.h_prev and the residual
  // sum, then the Table 1 update; pol.h_cur is not read)
  int policy;
  PolicyArgs pol;
};
// Small tensors (encode_is_small: rows * roundup(k/4, 64) <= 4096) are
// encoded in one launch that takes the amax itself (a.partial is not read);
// otherwise a.partial holds the amax partials of launch_amax_partial(_op).
bool encode_is_small(int64_t rows, int64_t k);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t s);
// The partial maxima of the epilogue tensor v = op(z, resid) of a.
hipError_t launch_amax_partial_op(const EncodeArgs &a, float *partial, int n_partial, hipStream_t s);
// RESIDUAL_RMSNORM: the per-row scales c = 1 / sqrt(sum u^2 / k + eps) of
// u = resid + z into a.rowscale (fixed-order fp64 sums).
hipError_t launch_rowscale(const EncodeArgs &a, hipStream_t s);
constexpr double kRmsEps = 1e-5;   // RMSNorm epsilon of the RESIDUAL_RMSNORM epilogue

// Weight-mask selection ([AE] App. E, Alg. 1 allocation with H = I).
hipError_t launch_select_mask(const float *w, int64_t rows, int64_t k, int32_t budget,
                              const float *partial, int n_partial, double *row_gain,
                              double *col_gain, uint8_t *mask_out, int fmt, const double *hdiag,
                              hipStream_t s);

// ---- gemv.hip ----
struct LinearArgs {
  // weight operand
  const uint8_t *w_codes, *w_scales, *w_mask, *w_offsets;
  const float *w_T;
  int32_t n_refined;
  int64_t n;                    // weight rows (outputs)
  // activation operand
  const uint8_t *x_codes, *x_scales, *x_offsets;
  const float *x_T;
  int64_t b;                    // tokens
  int64_t k;
  // level
  int32_t bits;
  const int32_t *bits_dev;
  float c2;
  int32_t waves;                // GEMV wavefronts per tile requested (0 = automatic)
  int32_t wk;                   // GEMV wavefronts per tile chosen at launch
  // output
  void *y;
  int y_dtype;
  // scratch
  _Float16 *xh;                 // dequantized activations [b][kpad]
  int64_t kpad;
  int32_t *prefix;              // weight-mask prefix table (GEMM)
  // per-token levels ([b] int32 device, 2/4/6) or null: one level for the call
  const int32_t *bits_rows;
  // batched GEMV: fp32 partial tiles of the K splits ([splits][b][n]) and their count
  float *part;
  int32_t splits;
  // element / offset format of both operands (autofp_format)
  int32_t fmt;
};
int64_t xh_kpad(int64_t k);
hipError_t launch_act_dequant(const LinearArgs &a, hipStream_t s);
bool gemv_needs_panel(const LinearArgs &a);   // true when the GEMV reads the fp16 activation panel
bool gemv_small_m_route(const LinearArgs &a);   // 17-64 tokens on the 64-token GEMM tile
bool gemv_panel_packed(const LinearArgs &a);    // 17+ tokens: panel kernel on packed activations
hipError_t launch_gemv(const LinearArgs &a, hipStream_t s);

// ---- gemv_batch.hip ----
// Batched decode GEMV, 17-64 tokens per slice (and every call with per-token
// levels): K % 128 == 0. Reads a.prefix at level 6 (or a device/per-token
// level) and a.part when the K range is split.
bool gemv_batch_ok(const LinearArgs &a);
// 9-64 tokens served by the batched kernel (gemv_batch_ok and the 9-16-token shape rule)
bool gemv_batch_route(const LinearArgs &a);
int64_t gemv_batch_part_floats(int64_t tokens);   // floats of a.part the launcher may use
hipError_t launch_gemv_batch(const LinearArgs &a, hipStream_t s);

// ---- gemm.hip ----
hipError_t launch_gemm(const LinearArgs &a, hipStream_t s);
bool gemm_small_m_ok(const LinearArgs &a);   // the 64-token GEMM tile applies (K % 64 == 0)
hipError_t launch_gemm_small_m(const LinearArgs &a, hipStream_t s);   // reads a.xh and, at level 6, a.prefix
// The variant formats (a.fmt != AUTOFP6) at any level, K % 64 == 0: writes
// the fp16 activation panel a.xh and (offset formats) the mask prefix
// a.prefix into the workspace when its kernels read them, then Y.
hipError_t launch_gemm_fmt(const LinearArgs &a, hipStream_t s);

// ---- gptq.hip ----
// Refinement-aware GPTQ ([AE] App. E, Algorithm 1) of w [rows][k] fp32 with the
// inverse-Hessian factor u [k][k] and the Hessian diagonal hdiag [k]; writes
// out's codes, scales, tensor scale, mask and offsets. Arguments checked by
// the caller; ws of gptq_workspace_bytes(rows, k).
size_t gptq_workspace_bytes(int64_t rows, int64_t k);
hipError_t launch_gptq(const float *w, int64_t rows, int64_t k, const double *u, const double *hdiag,
                       int32_t budget, const autofp_packed *out, void *ws, hipStream_t s);

// ---- signals.hip ----
int64_t entropy_slices(int64_t vocab);                        // vocabulary slices per row
size_t entropy_workspace_bytes(int64_t batch, int64_t vocab);  // per-slice candidates / partials
hipError_t launch_entropy(const float *logits, int64_t batch, int64_t vocab, int top_k,
                          float *out, void *workspace, hipStream_t s);
hipError_t launch_policy_update(const PolicyArgs &a, hipStream_t s);
hipError_t launch_policy_layer(const PolicyArgs &a, hipStream_t s);
hipError_t launch_update_norm(const void *h_prev, const void *h_cur, int dtype, int64_t batch,
                              int64_t hidden, float eps, float *out, hipStream_t s);

// ---- kv.hip ----
struct KvWriteArgs {
  const void *k, *v;
  int dtype;
  int64_t n_tokens;
  int h_kv;
  const int32_t *slots;
  int n_pages;
  uint8_t *k_pages, *v_pages;
  const uint8_t *page_kind;
  float *k_scale, *v_scale;
  int set_scale;                 // fold the partial maxima into new tensor scales
  const float *k_part, *v_part;  // amax partials of k and v (set_scale)
  int n_part;
};
hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t s);

struct KvAttnArgs {
  const void *q;
  int q_dtype;
  int64_t batch;
  int h_q, h_kv, grp;            // grp = h_q / h_kv query heads per KV head
  const uint8_t *k_pages, *v_pages, *page_kind;
  const float *k_scale, *v_scale;
  const int32_t *page_table, *seq_pages, *page_tokens;
  int n_pages, max_pages;
  int bits;
  const int32_t *bits_dev;
  float sm_scale;
  float *part;                   // [batch * h_q][n_split][kHd + 4] split records
  int n_split;
  float *out;
};
int kv_attn_splits(int64_t rows, int64_t max_pages);
int64_t kv_attn_max_pages();
size_t kv_attn_workspace_bytes(int64_t rows, int64_t max_pages);
hipError_t launch_kv_attention(const KvAttnArgs &a, hipStream_t s);

}  // namespace afp
