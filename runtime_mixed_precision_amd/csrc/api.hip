// C ABI of libautofp (declared in include/autofp.h): argument checks,
// workspace carving and kernel dispatch. No allocation, no synchronization.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>

#include "afp_launch.h"
#include "autofp.h"

using namespace afp;

static_assert(sizeof(autofp_policy_state) == 48, "policy state layout");
static_assert(sizeof(autofp_params) == 56, "params layout");

// Bytes of the static scratch array of autofp_quantize_noalloc (below).
constexpr size_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;
// bytes past the last row of a weight's offsets that the GEMV may read (never writes)
constexpr size_t kOffsetPad = 16;
// rows of autofp_gptq_quantize (16-row propagation blocks on grid.y)
constexpr int64_t kMaxGptqRows = 65535 * 16;
// largest reduction dimension of autofp_gemv / autofp_gemm
constexpr int64_t kMaxLinearK = (int64_t)1 << 22;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }

bool valid_k(int64_t k) { return k >= 16 && (k % 16) == 0; }

bool valid_format(int32_t f) { return f >= AUTOFP_FMT_AUTOFP6 && f <= AUTOFP_FMT_FP6G; }

// bytes per refined subgroup's offsets
int64_t offset_width(int32_t f) { return f == AUTOFP_FMT_AUTOFP8 ? 2 : 1; }

autofp_status from_hip(hipError_t e) { return e == hipSuccess ? AUTOFP_OK : AUTOFP_ERR_HIP; }

autofp_params params_or_default(const autofp_params *p) {
  autofp_params d;
  autofp_default_params(&d);
  return p ? *p : d;
}

int32_t refined_budget(int64_t k, double rho) {
  double r = floor(rho * (double)k / 4.0);
  const double cap = 2.0 * (double)(k / 16);
  if (r > cap) r = cap;
  if (r < 0) r = 0;
  return (int32_t)r;
}

// workspace pieces
size_t ws_quantize(int64_t rows, int64_t k) {
  (void)rows;
  return align_up(sizeof(float) * kAmaxBlocks) + align_up(sizeof(int32_t) * (mask_bytes(k) + 1));
}

// the epilogue's: the encode's, then one fp32 RMSNorm scale per row
size_t ws_epilogue(int64_t rows, int64_t k) { return ws_quantize(rows, k) + align_up(sizeof(float) * (size_t)rows); }

size_t ws_select(int64_t rows, int64_t k) {
  const size_t ncol = (size_t)(k / 4), ng = (size_t)(k / 16);
  return align_up(sizeof(float) * kAmaxBlocks) + align_up(sizeof(double) * (size_t)rows * ncol) +
         align_up(sizeof(double) * (ncol + 2 * ng) + sizeof(int32_t) * 4 * ng);
}

// fp16 activation panel, weight-mask prefix table, split-K partial tiles of
// the batched GEMV
size_t ws_linear(int64_t tokens, int64_t k) {
  return align_up(sizeof(_Float16) * (size_t)tokens * (size_t)xh_kpad(k)) +
         align_up(sizeof(int32_t) * (mask_bytes(k) + 1)) +
         align_up(sizeof(float) * (size_t)gemv_batch_part_floats(tokens));
}

size_t ws_kv_write() { return 2 * align_up(sizeof(float) * kAmaxBlocks); }

autofp_status check_kv_cache(const autofp_kv_cache *c) {
  if (!c) return AUTOFP_ERR_NULL;
  if (!c->k_pages || !c->v_pages || !c->page_kind || !c->k_scale || !c->v_scale) return AUTOFP_ERR_NULL;
  if (c->head_dim != AUTOFP_KV_HEAD_DIM || c->h_kv < 1 || c->h_kv > 65535 || c->n_pages < 1)
    return AUTOFP_ERR_SHAPE;
  if (!aligned16(c->k_pages) || !aligned16(c->v_pages)) return AUTOFP_ERR_ARG;
  return AUTOFP_OK;
}

autofp_status check_packed(const autofp_packed *t, int32_t kind) {
  if (!t) return AUTOFP_ERR_NULL;
  if (t->kind != kind) return AUTOFP_ERR_KIND;
  if (t->rows < 1 || !valid_k(t->k)) return AUTOFP_ERR_SHAPE;
  if (!t->codes || !t->scales || !t->tensor_scale) return AUTOFP_ERR_NULL;
  if (!aligned16(t->codes) || !aligned16(t->scales) || !aligned16(t->tensor_scale) ||
      (t->mask && !aligned16(t->mask)) || (t->offsets && !aligned16(t->offsets)))
    return AUTOFP_ERR_ARG;
  if (kind == AUTOFP_WEIGHT && (t->n_refined < 0 || t->n_refined > 2 * (t->k / 16)))
    return AUTOFP_ERR_ARG;
  if (!valid_format(t->format)) return AUTOFP_ERR_ARG;
  return AUTOFP_OK;
}

bool has_refinement(const autofp_packed *w, const autofp_packed *x) {
  const bool w_ok = w->mask != nullptr && (w->n_refined == 0 || w->offsets != nullptr);
  const bool x_ok = x->offsets != nullptr;
  return w_ok && x_ok;
}

autofp_status linear_common(const autofp_packed *w, const autofp_packed *x, int32_t bits,
                            const int32_t *bits_dev, void *y, int32_t y_dtype,
                            const autofp_params *p, void *ws, size_t ws_bytes, LinearArgs &a) {
  autofp_status st = check_packed(w, AUTOFP_WEIGHT);
  if (st != AUTOFP_OK) return st;
  st = check_packed(x, AUTOFP_ACTIVATION);
  if (st != AUTOFP_OK) return st;
  if (w->k != x->k) return AUTOFP_ERR_SHAPE;
  if (w->format != x->format) return AUTOFP_ERR_ARG;
  // the GEMM addresses one tile's fp16 activation rows ([256][round_up(k, 256)])
  // with 32-bit buffer offsets
  if (x->k > kMaxLinearK) return AUTOFP_ERR_SHAPE;
  if (!y) return AUTOFP_ERR_NULL;
  if (!aligned16(y)) return AUTOFP_ERR_ARG;
  if (y_dtype != AUTOFP_F32 && y_dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
  const int32_t fmt = w->format;
  if (fmt == AUTOFP_FMT_FP6G) {
    // the comparator format has one level and no refinement
    if (bits_dev || bits != 6) return AUTOFP_ERR_BITS;
  } else {
    if (!bits_dev && bits != 2 && bits != 4 && bits != 6 && !(bits == 8 && fmt == AUTOFP_FMT_AUTOFP8))
      return AUTOFP_ERR_BITS;
    if ((bits_dev || bits >= 6) && !has_refinement(w, x)) return AUTOFP_ERR_MISSING_REFINEMENT;
  }
  if (p && p->gemv_waves != 0 && p->gemv_waves != 1 && p->gemv_waves != 2 && p->gemv_waves != 4 &&
      p->gemv_waves != 8 && p->gemv_waves != 16)
    return AUTOFP_ERR_ARG;
  const size_t need = ws_linear(x->rows, x->k);
  if (!ws || ws_bytes < need) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(ws)) return AUTOFP_ERR_ARG;
  const autofp_params pp = params_or_default(p);
  a.w_codes = w->codes;
  a.w_scales = w->scales;
  a.w_mask = w->mask;
  a.w_offsets = w->offsets;
  a.w_T = w->tensor_scale;
  a.n_refined = w->n_refined;
  a.n = w->rows;
  a.x_codes = x->codes;
  a.x_scales = x->scales;
  a.x_offsets = x->offsets;
  a.x_T = x->tensor_scale;
  a.b = x->rows;
  a.k = x->k;
  a.bits = bits;
  a.bits_dev = bits_dev;
  a.c2 = pp.c2;
  a.waves = pp.gemv_waves;
  a.y = y;
  a.y_dtype = y_dtype;
  a.kpad = xh_kpad(x->k);
  a.xh = (_Float16 *)ws;
  a.prefix = (int32_t *)((char *)ws + align_up(sizeof(_Float16) * (size_t)x->rows * (size_t)a.kpad));
  a.part = (float *)((char *)a.prefix + align_up(sizeof(int32_t) * (mask_bytes(x->k) + 1)));
  a.splits = 1;
  a.bits_rows = nullptr;
  a.fmt = fmt;
  return AUTOFP_OK;
}

// A call that needs a variant format's own decode (levels above 4, or a
// level read on the device): it runs on the format-generic GEMM tiles.
bool variant_route(const LinearArgs &a) { return a.fmt != AUTOFP_FMT_AUTOFP6 && (a.bits_dev || a.bits >= 6); }

autofp_status launch_variant(const LinearArgs &a, hipStream_t s) {
  if (a.k % 64 != 0) return AUTOFP_ERR_SHAPE;
  return from_hip(launch_gemm_fmt(a, s));
}

// autofp_gemv's launches for arguments that linear_common accepted.
autofp_status gemv_launches(LinearArgs &a, const autofp_packed *w, const autofp_packed *x, int32_t bits,
                            const int32_t *bits_dev, hipStream_t s) {
  if (variant_route(a)) return launch_variant(a, s);
  if ((bits_dev || bits == 6) && x->rows <= 16 && x->k > 65536) return AUTOFP_ERR_SHAPE;
  if (gemv_needs_panel(a)) {
    const hipError_t e = launch_act_dequant(a, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  // the weight mask's prefix table, read by the 64-token GEMM tile (the
  // batched kernel forms its slice of it in each block)
  if (w->mask && (bits_dev || bits == 6) && gemv_small_m_route(a)) {
    const hipError_t e = launch_mask_prefix(w->mask, mask_bytes(w->k), a.prefix, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  return from_hip(launch_gemv(a, s));
}


autofp_status check_quantize(const void *x, int32_t x_dtype, int32_t refine, const uint8_t *exclude_mask,
                             const autofp_packed *out) {
  if (!x || !out) return AUTOFP_ERR_NULL;
  if (x_dtype != AUTOFP_F32 && x_dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
  if (out->kind != AUTOFP_WEIGHT && out->kind != AUTOFP_ACTIVATION) return AUTOFP_ERR_KIND;
  if (out->rows < 1 || !valid_k(out->k)) return AUTOFP_ERR_SHAPE;
  if (!out->codes || !out->scales || !out->tensor_scale) return AUTOFP_ERR_NULL;
  if (!aligned16(x) || !aligned16(out->codes) || !aligned16(out->scales) ||
      !aligned16(out->tensor_scale) || (out->mask && !aligned16(out->mask)) ||
      (out->offsets && !aligned16(out->offsets)) || (exclude_mask && !aligned16(exclude_mask)))
    return AUTOFP_ERR_ARG;
  if (!valid_format(out->format)) return AUTOFP_ERR_ARG;
  if (out->format == AUTOFP_FMT_FP6G && (refine || out->mask)) return AUTOFP_ERR_ARG;
  const bool act_refine = out->kind == AUTOFP_ACTIVATION && refine;
  const bool w_refine = out->kind == AUTOFP_WEIGHT && out->mask != nullptr;
  if (act_refine && (!out->mask || !out->offsets)) return AUTOFP_ERR_MISSING_REFINEMENT;
  if (out->kind == AUTOFP_WEIGHT && refine && !out->mask) return AUTOFP_ERR_MISSING_REFINEMENT;
  if (w_refine) {
    if (out->n_refined < 0 || out->n_refined > 2 * (out->k / 16)) return AUTOFP_ERR_ARG;
    if (out->n_refined > 0 && !out->offsets) return AUTOFP_ERR_MISSING_REFINEMENT;
  }
  return AUTOFP_OK;
}

// The encode's arguments on scratch `ws` (ws_quantize bytes: amax partials,
// then the weight-mask prefix table); arguments already checked. `epi`
// (op != 0) encodes the producer epilogue's v instead of x.
EncodeArgs encode_args(const void *x, int32_t x_dtype, int32_t refine, const uint8_t *exclude_mask,
                       const autofp_params *p, const autofp_packed *out, void *ws, const EncodeArgs *epi) {
  const autofp_params pp = params_or_default(p);
  const bool act_refine = out->kind == AUTOFP_ACTIVATION && refine;
  const bool w_refine = out->kind == AUTOFP_WEIGHT && out->mask != nullptr;
  EncodeArgs a{};
  if (epi) {
    a.op = epi->op;
    a.z = epi->z;
    a.ldz = epi->ldz;
    a.resid = epi->resid;
    a.v_out = epi->v_out;
    a.rowscale = epi->rowscale;
    a.policy = epi->policy;
    a.pol = epi->pol;
  }
  a.rows = out->rows;
  a.k = out->k;
  a.x = x;
  a.dtype = x_dtype;
  a.partial = (float *)ws;
  a.n_partial = amax_partial_count(out->rows * out->k);
  a.codes = out->codes;
  a.scales = out->scales;
  a.tensor_scale = out->tensor_scale;
  a.act_refine = act_refine ? 1 : 0;
  a.exclude_mask = act_refine ? exclude_mask : nullptr;
  a.thresh = pp.act_nmse_thresh;
  a.act_mask = act_refine ? out->mask : nullptr;
  a.act_offsets = act_refine ? out->offsets : nullptr;
  a.w_mask = w_refine ? out->mask : nullptr;
  a.w_prefix = (int32_t *)((char *)ws + align_up(sizeof(float) * kAmaxBlocks));
  a.n_refined = out->n_refined;
  a.w_offsets = out->offsets;
  a.fmt = out->format;
  return a;
}

// The encode's launches (see encode_args).
autofp_status launch_quantize(const void *x, int32_t x_dtype, int32_t refine, const uint8_t *exclude_mask,
                              const autofp_params *p, const autofp_packed *out, void *ws, hipStream_t s,
                              const EncodeArgs *epi = nullptr) {
  const EncodeArgs a = encode_args(x, x_dtype, refine, exclude_mask, p, out, ws, epi);
  float *partial = (float *)ws;
  int32_t *prefix = (int32_t *)((char *)ws + align_up(sizeof(float) * kAmaxBlocks));
  hipError_t e = hipSuccess;
  if (!encode_is_small(out->rows, out->k)) {
    if (a.op == AUTOFP_EPI_RESIDUAL_RMSNORM) {
      e = launch_rowscale(a, s);
      if (e != hipSuccess) return AUTOFP_ERR_HIP;
    }
    e = a.op ? launch_amax_partial_op(a, partial, a.n_partial, s)
             : launch_amax_partial(x, x_dtype, out->rows * out->k, partial, a.n_partial, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  if (a.w_mask) {
    e = launch_mask_prefix(out->mask, mask_bytes(out->k), prefix, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  return from_hip(launch_encode(a, s));
}

// ---------------------------------------------------------------------------
// Scratch of autofp_quantize_noalloc: one file-scope device array. Every GPU
// the library runs on holds its own copy (at its own address) until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels. Calls on one GPU share the array, so calls that overlap
// in time on one GPU race; nothing in it needs to start at zero (each call
// writes every entry it reads before reading it).
// ---------------------------------------------------------------------------
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_dev[kScratchDevices];

autofp_status scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AUTOFP_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return AUTOFP_ERR_ARG;
  void *p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    // the same address on every concurrent first call: storing it twice is benign
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AUTOFP_ERR_HIP;
    g_scratch_dev[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return AUTOFP_OK;
}

}  // namespace

extern "C" {

autofp_status autofp_default_params(autofp_params *p) {
  if (!p) return AUTOFP_ERR_NULL;
  p->rho = 0.2;
  p->act_nmse_thresh = 0.003f;
  p->c2 = 2.0f;
  p->top_k = 10;
  p->eps = 1e-6f;
  p->tau = 0.10;
  p->lambda_d = 0.7;
  p->alpha = 4;
  p->beta = 2;
  p->n_p = 2;
  p->gemv_waves = 0;
  return AUTOFP_OK;
}

const char *autofp_status_string(autofp_status s) {
  switch (s) {
    case AUTOFP_OK: return "ok";
    case AUTOFP_ERR_NULL: return "null pointer";
    case AUTOFP_ERR_SHAPE: return "bad shape (k must be a positive multiple of 16)";
    case AUTOFP_ERR_BITS: return "precision level not in {2, 4, 6}";
    case AUTOFP_ERR_KIND: return "operand kind mismatch";
    case AUTOFP_ERR_WORKSPACE: return "workspace missing or too small";
    case AUTOFP_ERR_MISSING_REFINEMENT: return "level 6 needs masks and offsets";
    case AUTOFP_ERR_DTYPE: return "unsupported dtype";
    case AUTOFP_ERR_ARG: return "argument out of range or misaligned";
    case AUTOFP_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

autofp_status autofp_packed_bytes(int64_t rows, int64_t k, int32_t kind, int32_t format,
                                  int32_t refine, int32_t n_refined, size_t out_bytes[5]) {
  if (!out_bytes) return AUTOFP_ERR_NULL;
  if (rows < 1 || !valid_k(k)) return AUTOFP_ERR_SHAPE;
  if (kind != AUTOFP_WEIGHT && kind != AUTOFP_ACTIVATION) return AUTOFP_ERR_KIND;
  if (n_refined < 0 || n_refined > 2 * (k / 16)) return AUTOFP_ERR_ARG;
  if (!valid_format(format) || (format == AUTOFP_FMT_FP6G && refine)) return AUTOFP_ERR_ARG;
  const int64_t ow = offset_width(format);
  out_bytes[0] = (size_t)(rows * (format == AUTOFP_FMT_FP6G ? 3 * k / 4 : k / 2));
  out_bytes[1] = (size_t)(rows * (k / 16));
  out_bytes[2] = sizeof(float);
  out_bytes[3] = 0;
  out_bytes[4] = 0;
  if (refine) {
    if (kind == AUTOFP_WEIGHT) {
      out_bytes[3] = (size_t)mask_bytes(k);
      out_bytes[4] = (size_t)rows * (size_t)n_refined * (size_t)ow + kOffsetPad;
    } else {
      out_bytes[3] = (size_t)(rows * mask_bytes(k));
      out_bytes[4] = (size_t)(rows * (k / 4) * ow);
    }
  }
  return AUTOFP_OK;
}

autofp_status autofp_weight_refined_count(int64_t k, const autofp_params *p, int32_t *n_refined) {
  if (!p || !n_refined) return AUTOFP_ERR_NULL;
  if (!valid_k(k)) return AUTOFP_ERR_SHAPE;
  if (!(p->rho >= 0.0 && p->rho <= 1.0)) return AUTOFP_ERR_ARG;
  *n_refined = refined_budget(k, p->rho);
  return AUTOFP_OK;
}

autofp_status autofp_workspace_bytes(int32_t op, int64_t rows, int64_t k, size_t *bytes) {
  if (!bytes) return AUTOFP_ERR_NULL;
  if (op == AUTOFP_OP_KV_WRITE) {
    if (rows < 1 || k != AUTOFP_KV_HEAD_DIM) return AUTOFP_ERR_SHAPE;
    *bytes = ws_kv_write();
    return AUTOFP_OK;
  }
  if (op == AUTOFP_OP_KV_ATTENTION) {
    if (rows < 1 || k < 1 || k > kv_attn_max_pages()) return AUTOFP_ERR_SHAPE;
    *bytes = kv_attn_workspace_bytes(rows, k);
    return AUTOFP_OK;
  }
  if (op == AUTOFP_OP_SIGNALS) {
    if (rows < 1 || k < 1 || rows > 65535) return AUTOFP_ERR_SHAPE;
    *bytes = entropy_workspace_bytes(rows, k);
    return AUTOFP_OK;
  }
  if (rows < 1 || !valid_k(k)) return AUTOFP_ERR_SHAPE;
  switch (op) {
    case AUTOFP_OP_QUANTIZE: *bytes = ws_quantize(rows, k); return AUTOFP_OK;
    case AUTOFP_OP_SELECT_MASK:
      if (k > 65536) return AUTOFP_ERR_SHAPE;
      *bytes = ws_select(rows, k);
      return AUTOFP_OK;
    case AUTOFP_OP_GEMV:
    case AUTOFP_OP_GEMM: *bytes = ws_linear(rows, k); return AUTOFP_OK;
    case AUTOFP_OP_GPTQ:
      if (k > 65536 || rows > kMaxGptqRows) return AUTOFP_ERR_SHAPE;
      *bytes = gptq_workspace_bytes(rows, k);
      return AUTOFP_OK;
    case AUTOFP_OP_EPILOGUE: *bytes = ws_epilogue(rows, k); return AUTOFP_OK;
    default: return AUTOFP_ERR_ARG;
  }
}

autofp_status autofp_select_weight_mask(const float *w, int64_t rows, int64_t k, int32_t format,
                                        const autofp_params *p, uint8_t *mask_out, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  if (!w || !p || !mask_out) return AUTOFP_ERR_NULL;
  if (rows < 1 || !valid_k(k) || k > 65536) return AUTOFP_ERR_SHAPE;
  if (!(p->rho >= 0.0 && p->rho <= 1.0)) return AUTOFP_ERR_ARG;
  if (!valid_format(format) || format == AUTOFP_FMT_FP6G) return AUTOFP_ERR_ARG;
  if (!aligned16(w) || !aligned16(mask_out)) return AUTOFP_ERR_ARG;
  if (!workspace || workspace_bytes < ws_select(rows, k)) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return AUTOFP_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  float *partial = (float *)ws;
  ws += align_up(sizeof(float) * kAmaxBlocks);
  double *row_gain = (double *)ws;
  ws += align_up(sizeof(double) * (size_t)rows * (size_t)(k / 4));
  double *col_gain = (double *)ws;
  const int np = amax_partial_count(rows * k);
  hipError_t e = launch_amax_partial(w, AUTOFP_F32, rows * k, partial, np, s);
  if (e != hipSuccess) return AUTOFP_ERR_HIP;
  e = launch_select_mask(w, rows, k, refined_budget(k, p->rho), partial, np, row_gain, col_gain,
                         mask_out, format, nullptr, s);
  return from_hip(e);
}

autofp_status autofp_gptq_quantize(const float *w, int64_t rows, int64_t k, const double *u,
                                   const double *h_diag, const autofp_params *p, autofp_packed *out,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  if (!w || !u || !h_diag || !out) return AUTOFP_ERR_NULL;
  if (rows < 1 || !valid_k(k) || k > 65536 || rows > kMaxGptqRows) return AUTOFP_ERR_SHAPE;
  if (out->kind != AUTOFP_WEIGHT) return AUTOFP_ERR_KIND;
  if (out->rows != rows || out->k != k) return AUTOFP_ERR_SHAPE;
  if (!out->codes || !out->scales || !out->tensor_scale) return AUTOFP_ERR_NULL;
  if (!out->mask || !out->offsets) return AUTOFP_ERR_MISSING_REFINEMENT;
  const autofp_params pp = params_or_default(p);
  if (!(pp.rho >= 0.0 && pp.rho <= 1.0)) return AUTOFP_ERR_ARG;
  if (out->format != AUTOFP_FMT_AUTOFP6 || out->n_refined != refined_budget(k, pp.rho)) return AUTOFP_ERR_ARG;
  if (!aligned16(w) || !aligned16(u) || !aligned16(h_diag) || !aligned16(out->codes) || !aligned16(out->scales) ||
      !aligned16(out->tensor_scale) || !aligned16(out->mask) || !aligned16(out->offsets))
    return AUTOFP_ERR_ARG;
  if (!workspace || workspace_bytes < gptq_workspace_bytes(rows, k)) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return AUTOFP_ERR_ARG;
  return from_hip(launch_gptq(w, rows, k, u, h_diag, out->n_refined, out, workspace, (hipStream_t)stream));
}

autofp_status autofp_quantize(const void *x, int32_t x_dtype, int32_t refine,
                              const uint8_t *exclude_mask, const autofp_params *p,
                              autofp_packed *out, void *workspace, size_t workspace_bytes,
                              void *stream) {
  const autofp_status st = check_quantize(x, x_dtype, refine, exclude_mask, out);
  if (st != AUTOFP_OK) return st;
  if (!workspace || workspace_bytes < ws_quantize(out->rows, out->k)) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return AUTOFP_ERR_ARG;
  return launch_quantize(x, x_dtype, refine, exclude_mask, p, out, workspace, (hipStream_t)stream);
}

autofp_status autofp_epilogue_quantize(int32_t op, const float *z, int64_t ldz, const float *residual,
                                       float *v_out, int32_t refine, const uint8_t *exclude_mask,
                                       const autofp_params *p, autofp_packed *out, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  if (!z) return AUTOFP_ERR_NULL;
  if (op != AUTOFP_EPI_COPY && op != AUTOFP_EPI_RESIDUAL && op != AUTOFP_EPI_SWIGLU &&
      op != AUTOFP_EPI_RESIDUAL_RMSNORM)
    return AUTOFP_ERR_ARG;
  const bool resid_op = op == AUTOFP_EPI_RESIDUAL || op == AUTOFP_EPI_RESIDUAL_RMSNORM;
  if (resid_op && !residual) return AUTOFP_ERR_NULL;
  // the encode's own checks, with z standing in for the input pointer
  const autofp_status st = check_quantize(z, AUTOFP_F32, refine, exclude_mask, out);
  if (st != AUTOFP_OK) return st;
  if (out->kind != AUTOFP_ACTIVATION) return AUTOFP_ERR_KIND;
  if (ldz < (op == AUTOFP_EPI_SWIGLU ? 2 : 1) * out->k || (ldz & 3) != 0) return AUTOFP_ERR_SHAPE;
  if ((residual && !aligned16(residual)) || (v_out && !aligned16(v_out))) return AUTOFP_ERR_ARG;
  const size_t need = op == AUTOFP_EPI_RESIDUAL_RMSNORM ? ws_epilogue(out->rows, out->k) : ws_quantize(out->rows, out->k);
  if (!workspace || workspace_bytes < need) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return AUTOFP_ERR_ARG;
  EncodeArgs epi{};
  epi.op = op;
  epi.z = z;
  epi.ldz = ldz;
  epi.resid = resid_op ? residual : nullptr;
  epi.v_out = v_out;
  epi.rowscale = op == AUTOFP_EPI_RESIDUAL_RMSNORM
                     ? (float *)((char *)workspace + ws_quantize(out->rows, out->k))
                     : nullptr;
  return launch_quantize(z, AUTOFP_F32, refine, exclude_mask, p, out, workspace, (hipStream_t)stream, &epi);
}

autofp_status autofp_layer_epilogue(const float *z, int64_t ldz, const float *residual, float *v_out,
                                    const float *h_prev, int32_t refine, const uint8_t *exclude_mask,
                                    int32_t phase, int32_t layer, int32_t new_sequence, const float *g_e,
                                    const autofp_params *p, autofp_policy_state *state, float *l_a_out,
                                    int32_t *bits_rows, int32_t *bits_layer, autofp_packed *out,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  if (!z || !residual || !v_out || !h_prev || !l_a_out || !state || !bits_rows) return AUTOFP_ERR_NULL;
  const autofp_params pp = params_or_default(p);
  if (phase != 0 && phase != 1) return AUTOFP_ERR_ARG;
  if (phase == 1 && !g_e) return AUTOFP_ERR_NULL;
  if (layer < 0 || pp.alpha < 1 || pp.beta < 1 || pp.n_p < 1 ||
      !(pp.lambda_d >= 0.0 && pp.lambda_d <= 1.0) || !(pp.eps >= 0.0f))
    return AUTOFP_ERR_ARG;
  // the checks of autofp_epilogue_quantize with RESIDUAL_RMSNORM
  const autofp_status st = check_quantize(z, AUTOFP_F32, refine, exclude_mask, out);
  if (st != AUTOFP_OK) return st;
  if (out->kind != AUTOFP_ACTIVATION) return AUTOFP_ERR_KIND;
  if (ldz < out->k || (ldz & 3) != 0) return AUTOFP_ERR_SHAPE;
  if (!aligned16(residual) || !aligned16(v_out) || !aligned16(h_prev)) return AUTOFP_ERR_ARG;
  if ((const void *)h_prev == (const void *)v_out || (const void *)residual == (const void *)v_out)
    return AUTOFP_ERR_ARG;
  if (!workspace || workspace_bytes < ws_epilogue(out->rows, out->k)) return AUTOFP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return AUTOFP_ERR_ARG;
  PolicyArgs pa{};
  pa.phase = phase;
  pa.layer = layer;
  pa.new_sequence = new_sequence;
  pa.g_e = g_e;
  pa.batch = out->rows;
  pa.tau = pp.tau;
  pa.lambda_d = pp.lambda_d;
  pa.alpha = pp.alpha;
  pa.beta = pp.beta;
  pa.n_p = pp.n_p;
  pa.state = state;
  pa.bits_rows = bits_rows;
  pa.bits_layer = bits_layer;
  pa.h_prev = h_prev;
  pa.h_cur = v_out;
  pa.h_dtype = AUTOFP_F32;
  pa.hidden = out->k;
  pa.eps = pp.eps;
  pa.l_a_out = l_a_out;
  EncodeArgs epi{};
  epi.op = AUTOFP_EPI_RESIDUAL_RMSNORM;
  epi.z = z;
  epi.ldz = ldz;
  epi.resid = residual;
  epi.v_out = v_out;
  epi.rowscale = (float *)((char *)workspace + ws_quantize(out->rows, out->k));
  hipStream_t s = (hipStream_t)stream;
  if (encode_is_small(out->rows, out->k)) {
    epi.policy = 1;
    epi.pol = pa;
    return launch_quantize(z, AUTOFP_F32, refine, exclude_mask, p, out, workspace, s, &epi);
  }
  const autofp_status e = launch_quantize(z, AUTOFP_F32, refine, exclude_mask, p, out, workspace, s, &epi);
  if (e != AUTOFP_OK) return e;
  return from_hip(launch_policy_layer(pa, s));
}

autofp_status autofp_quantize_noalloc(const void *x, int32_t x_dtype, int32_t refine,
                                      const uint8_t *exclude_mask, const autofp_params *p,
                                      autofp_packed *out, void *stream) {
  const autofp_status st = check_quantize(x, x_dtype, refine, exclude_mask, out);
  if (st != AUTOFP_OK) return st;
  if (ws_quantize(out->rows, out->k) > kScratchBytes) return AUTOFP_ERR_WORKSPACE;
  void *ws = nullptr;
  const autofp_status ss = scratch_ptr(&ws);
  if (ss != AUTOFP_OK) return ss;
  return launch_quantize(x, x_dtype, refine, exclude_mask, p, out, ws, (hipStream_t)stream);
}

autofp_status autofp_gemv(const autofp_packed *w, const autofp_packed *x, int32_t bits,
                          const int32_t *bits_dev, void *y, int32_t y_dtype,
                          const autofp_params *p, void *workspace, size_t workspace_bytes,
                          void *stream) {
  LinearArgs a{};
  const autofp_status st =
      linear_common(w, x, bits, bits_dev, y, y_dtype, p, workspace, workspace_bytes, a);
  if (st != AUTOFP_OK) return st;
  return gemv_launches(a, w, x, bits, bits_dev, (hipStream_t)stream);
}

autofp_status autofp_gemv_rows(const autofp_packed *w, const autofp_packed *x, const int32_t *bits_rows,
                               void *y, int32_t y_dtype, const autofp_params *p, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (!bits_rows) return AUTOFP_ERR_NULL;
  if (!aligned16(bits_rows)) return AUTOFP_ERR_ARG;
  LinearArgs a{};
  // every row may run at level 6: both operands must carry their refinement
  const autofp_status st =
      linear_common(w, x, 4, bits_rows, y, y_dtype, p, workspace, workspace_bytes, a);
  if (st != AUTOFP_OK) return st;
  if (a.fmt != AUTOFP_FMT_AUTOFP6) return AUTOFP_ERR_ARG;
  if (x->k % 128 != 0) return AUTOFP_ERR_SHAPE;
  a.bits_dev = nullptr;
  a.bits_rows = bits_rows;
  if (!gemv_batch_ok(a)) return AUTOFP_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  return from_hip(launch_gemv_batch(a, s));   // the kernel forms the mask prefix itself
}

autofp_status autofp_gemm(const autofp_packed *w, const autofp_packed *x, int32_t bits,
                          const int32_t *bits_dev, void *y, int32_t y_dtype,
                          const autofp_params *p, void *workspace, size_t workspace_bytes,
                          void *stream) {
  LinearArgs a{};
  const autofp_status st =
      linear_common(w, x, bits, bits_dev, y, y_dtype, p, workspace, workspace_bytes, a);
  if (st != AUTOFP_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (variant_route(a)) return launch_variant(a, s);
  hipError_t e = launch_act_dequant(a, s);
  if (e != hipSuccess) return AUTOFP_ERR_HIP;
  if (w->mask && (bits_dev || bits == 6)) {
    e = launch_mask_prefix(w->mask, mask_bytes(w->k), a.prefix, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  return from_hip(launch_gemm(a, s));
}

autofp_status autofp_policy_signals(const float *logits, int64_t batch, int64_t vocab,
                                    const void *h_prev, const void *h_cur, int32_t h_dtype,
                                    int64_t hidden, const autofp_params *p, float *entropy_out,
                                    float *update_out, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  const autofp_params pp = params_or_default(p);
  if (!entropy_out && !update_out) return AUTOFP_ERR_NULL;
  if (batch < 1) return AUTOFP_ERR_SHAPE;
  if (entropy_out) {
    if (!logits) return AUTOFP_ERR_NULL;
    if (vocab < 1) return AUTOFP_ERR_SHAPE;
    if (pp.top_k < 1 || (pp.top_k > 32 && pp.top_k < vocab)) return AUTOFP_ERR_ARG;
    if (!aligned16(logits)) return AUTOFP_ERR_ARG;
    if (batch > 65535) return AUTOFP_ERR_SHAPE;
    if (!workspace || !aligned16(workspace) || workspace_bytes < entropy_workspace_bytes(batch, vocab))
      return AUTOFP_ERR_WORKSPACE;
  }
  if (update_out) {
    if (!h_prev || !h_cur) return AUTOFP_ERR_NULL;
    if (hidden < 1) return AUTOFP_ERR_SHAPE;
    if (h_dtype != AUTOFP_F32 && h_dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
    if (!(pp.eps >= 0.0f)) return AUTOFP_ERR_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  if (entropy_out) {
    const hipError_t e = launch_entropy(logits, batch, vocab, pp.top_k, entropy_out, workspace, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  if (update_out) {
    const hipError_t e = launch_update_norm(h_prev, h_cur, h_dtype, batch, hidden, pp.eps, update_out, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
  }
  return AUTOFP_OK;
}

autofp_status autofp_policy_update(int32_t phase, int32_t layer, int32_t new_sequence,
                                   const float *l_a, const float *g_e, int64_t batch,
                                   const autofp_params *p, autofp_policy_state *state,
                                   int32_t *bits_rows, int32_t *bits_layer, void *stream) {
  const autofp_params pp = params_or_default(p);
  if (!l_a || !state || !bits_rows) return AUTOFP_ERR_NULL;
  if (phase != 0 && phase != 1) return AUTOFP_ERR_ARG;
  if (phase == 1 && !g_e) return AUTOFP_ERR_NULL;
  if (batch < 1) return AUTOFP_ERR_SHAPE;
  if (layer < 0 || pp.alpha < 1 || pp.beta < 1 || pp.n_p < 1 ||
      !(pp.lambda_d >= 0.0 && pp.lambda_d <= 1.0))
    return AUTOFP_ERR_ARG;
  PolicyArgs a{};
  a.phase = phase;
  a.layer = layer;
  a.new_sequence = new_sequence;
  a.l_a = l_a;
  a.g_e = g_e;
  a.batch = batch;
  a.tau = pp.tau;
  a.lambda_d = pp.lambda_d;
  a.alpha = pp.alpha;
  a.beta = pp.beta;
  a.n_p = pp.n_p;
  a.state = state;
  a.bits_rows = bits_rows;
  a.bits_layer = bits_layer;
  return from_hip(launch_policy_update(a, (hipStream_t)stream));
}

autofp_status autofp_policy_layer(int32_t phase, int32_t layer, int32_t new_sequence,
                                  const void *h_prev, const void *h_cur, int32_t h_dtype,
                                  int64_t hidden, const float *g_e, int64_t batch,
                                  const autofp_params *p, autofp_policy_state *state,
                                  float *l_a_out, int32_t *bits_rows, int32_t *bits_layer,
                                  void *stream) {
  const autofp_params pp = params_or_default(p);
  if (!h_prev || !h_cur || !l_a_out || !state || !bits_rows) return AUTOFP_ERR_NULL;
  if (phase != 0 && phase != 1) return AUTOFP_ERR_ARG;
  if (phase == 1 && !g_e) return AUTOFP_ERR_NULL;
  if (batch < 1 || hidden < 1) return AUTOFP_ERR_SHAPE;
  if (h_dtype != AUTOFP_F32 && h_dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
  if (layer < 0 || pp.alpha < 1 || pp.beta < 1 || pp.n_p < 1 ||
      !(pp.lambda_d >= 0.0 && pp.lambda_d <= 1.0) || !(pp.eps >= 0.0f))
    return AUTOFP_ERR_ARG;
  PolicyArgs a{};
  a.phase = phase;
  a.layer = layer;
  a.new_sequence = new_sequence;
  a.g_e = g_e;
  a.batch = batch;
  a.tau = pp.tau;
  a.lambda_d = pp.lambda_d;
  a.alpha = pp.alpha;
  a.beta = pp.beta;
  a.n_p = pp.n_p;
  a.state = state;
  a.bits_rows = bits_rows;
  a.bits_layer = bits_layer;
  a.h_prev = h_prev;
  a.h_cur = h_cur;
  a.h_dtype = h_dtype;
  a.hidden = hidden;
  a.eps = pp.eps;
  a.l_a_out = l_a_out;
  return from_hip(launch_policy_layer(a, (hipStream_t)stream));
}

autofp_status autofp_kv_write(const void *k, const void *v, int32_t dtype, int64_t n_tokens,
                              const int32_t *slots, int32_t set_scale,
                              const autofp_kv_cache *cache, void *workspace,
                              size_t workspace_bytes, void *stream) {
  if (!k || !v || !slots) return AUTOFP_ERR_NULL;
  const autofp_status cs = check_kv_cache(cache);
  if (cs != AUTOFP_OK) return cs;
  if (n_tokens < 1 || n_tokens * cache->h_kv > ((int64_t)1 << 40) / AUTOFP_KV_HEAD_DIM)
    return AUTOFP_ERR_SHAPE;
  if (dtype != AUTOFP_F32 && dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
  if (!aligned16(k) || !aligned16(v)) return AUTOFP_ERR_ARG;
  KvWriteArgs a{};
  a.k = k;
  a.v = v;
  a.dtype = dtype;
  a.n_tokens = n_tokens;
  a.h_kv = cache->h_kv;
  a.slots = slots;
  a.n_pages = cache->n_pages;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.page_kind = cache->page_kind;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.set_scale = set_scale != 0;
  hipStream_t s = (hipStream_t)stream;
  if (a.set_scale) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < ws_kv_write()) return AUTOFP_ERR_WORKSPACE;
    float *kp = (float *)workspace;
    float *vp = (float *)((char *)workspace + align_up(sizeof(float) * kAmaxBlocks));
    const int64_t n = n_tokens * cache->h_kv * AUTOFP_KV_HEAD_DIM;
    const int np = amax_partial_count(n);
    hipError_t e = launch_amax_partial(k, dtype, n, kp, np, s);
    if (e == hipSuccess) e = launch_amax_partial(v, dtype, n, vp, np, s);
    if (e != hipSuccess) return AUTOFP_ERR_HIP;
    a.k_part = kp;
    a.v_part = vp;
    a.n_part = np;
  }
  return from_hip(launch_kv_write(a, s));
}

autofp_status autofp_kv_attention(const void *q, int32_t q_dtype, int64_t batch, int32_t h_q,
                                  const autofp_kv_cache *cache, int32_t bits,
                                  const int32_t *bits_dev, float sm_scale, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !out) return AUTOFP_ERR_NULL;
  const autofp_status cs = check_kv_cache(cache);
  if (cs != AUTOFP_OK) return cs;
  if (!cache->page_table || !cache->seq_pages || !cache->page_tokens) return AUTOFP_ERR_NULL;
  if (batch < 1 || batch > 65535 || h_q < 1 || h_q % cache->h_kv != 0 || h_q / cache->h_kv > 16)
    return AUTOFP_ERR_SHAPE;
  if (cache->max_pages < 1 || cache->max_pages > kv_attn_max_pages()) return AUTOFP_ERR_SHAPE;
  if (!bits_dev && bits != 2 && bits != 4 && bits != 6) return AUTOFP_ERR_BITS;
  if (q_dtype != AUTOFP_F32 && q_dtype != AUTOFP_BF16) return AUTOFP_ERR_DTYPE;
  if (!isfinite(sm_scale)) return AUTOFP_ERR_ARG;
  if (!aligned16(q) || !aligned16(out)) return AUTOFP_ERR_ARG;
  const int64_t rows = batch * h_q;
  if (!workspace || !aligned16(workspace) || workspace_bytes < kv_attn_workspace_bytes(rows, cache->max_pages))
    return AUTOFP_ERR_WORKSPACE;
  KvAttnArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = batch;
  a.h_q = h_q;
  a.h_kv = cache->h_kv;
  a.grp = h_q / cache->h_kv;
  a.k_pages = cache->k_pages;
  a.v_pages = cache->v_pages;
  a.page_kind = cache->page_kind;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.page_table = cache->page_table;
  a.seq_pages = cache->seq_pages;
  a.page_tokens = cache->page_tokens;
  a.n_pages = cache->n_pages;
  a.max_pages = cache->max_pages;
  a.bits = bits;
  a.bits_dev = bits_dev;
  a.sm_scale = sm_scale;
  a.part = (float *)workspace;
  a.n_split = kv_attn_splits(rows, cache->max_pages);
  a.out = out;
  return from_hip(launch_kv_attention(a, (hipStream_t)stream));
}

}  // extern "C"
