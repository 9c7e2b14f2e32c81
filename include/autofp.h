/*
 * autofp.h - C ABI of the AutoFP block-scaled low-bit linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * Source of the method: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM
 * Inference via Automatic Exponent-Mantissa Refinement" (arXiv 2611.10165v1),
 * cited below as [AE] with the section, equation, table or figure.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory. Every data pointer is DEVICE memory owned by the caller unless the
 *    argument says "host". The library never allocates, frees or synchronizes;
 *    scratch space comes from the caller through (workspace, workspace_bytes),
 *    sized by autofp_workspace_bytes(). Device pointers need 16-byte alignment.
 *  - Streams. `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream). Calls are asynchronous on it; the returned status reports
 *    argument checks and the launch result only, never kernel completion.
 *  - Errors. Arguments are checked before anything is launched; on any error
 *    nothing is launched and no output is written.
 *  - Shapes. A tensor is [rows x k] row-major with k the reduction dimension;
 *    k must be a positive multiple of 16 (one NVFP4 group, [AE] App. B.1).
 *  - Non-finite inputs (inf / NaN) give unspecified results.
 *  - Thread safety: concurrent calls on different buffers are safe. The only
 *    process-wide state is a cache of device properties (each entry set once,
 *    atomically) and the static scratch of autofp_quantize_noalloc (calls of
 *    it that overlap on one GPU race; see there).
 */
#ifndef AUTOFP_H
#define AUTOFP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AUTOFP_OK = 0,
  AUTOFP_ERR_NULL = 1,               /* a required pointer is NULL                  */
  AUTOFP_ERR_SHAPE = 2,              /* k % 16 != 0, rows < 1, mismatched shapes    */
  AUTOFP_ERR_BITS = 3,               /* level not in {2, 4, 6} (8: AutoFP8 only)    */
  AUTOFP_ERR_KIND = 4,               /* weight/activation operand in the wrong slot */
  AUTOFP_ERR_WORKSPACE = 5,          /* workspace NULL or smaller than required     */
  AUTOFP_ERR_MISSING_REFINEMENT = 6, /* level 6 without mask/offsets                */
  AUTOFP_ERR_DTYPE = 7,              /* unsupported dtype code                      */
  AUTOFP_ERR_ARG = 8,                /* a parameter out of its documented range     */
  AUTOFP_ERR_HIP = 9                 /* the HIP runtime reported a launch error     */
} autofp_status;

typedef enum { AUTOFP_F32 = 0, AUTOFP_BF16 = 1 } autofp_dtype;
typedef enum { AUTOFP_WEIGHT = 0, AUTOFP_ACTIVATION = 1 } autofp_kind;

/*
 * Element and offset format of a packed tensor (autofp_packed.format). The
 * first three share the NVFP4 base (E2M1 codes, E4M3 group scales, FP32
 * tensor scale) and the subgroup masks; they differ in the signed offsets d
 * of the refined subgroups and their value delta:
 *  AUTOFP6   d in {-2,-1,0,+1}, delta = d/8, 2 bits per element, one byte per
 *            subgroup ([AE] §3.2). The default (zero).
 *  AUTOFP6E  d in {-2,-1,0,+1}, delta = d * 2^(e-3) with e the unbiased
 *            exponent of the element's E2M1 value q (0 for |q| < 1, 1 for
 *            2 and 3, 2 for 4 and 6): the exponent-scaled offset step that
 *            [AE] §6.5 / Fig. 14(a) compares with the fixed one. Same storage
 *            as AUTOFP6.
 *  AUTOFP8   d in {-8..7}, delta = d/8, 4 bits per element, two bytes per
 *            subgroup, element e of the subgroup in bits [4e+3:4e] of the
 *            little-endian 16-bit word ([AE] App. I, Table 10: offsets widened
 *            from 2 to 4 bits; 5.3 bits per weight at rho = 0.2). Runs at
 *            level 8 with d, and at level 6 with d clamped to [-2, +1] (the
 *            AutoFP6 offset of the same element).
 *  FP6G      the group-scaled 6-bit comparator of [AE] App. B.2: E2M3
 *            elements (bias 1, maximum 7.5) under the NVFP4 scaling hierarchy,
 *            T = amax/(7.5*448), B_j = E4M3(amax_j/(7.5 T)). Codes [rows][3k/4]:
 *            four 6-bit codes s|e1|e0|m2|m1|m0 per three bytes, code i of a
 *            subgroup at bits [6i+5:6i] of the little-endian 24-bit word. No
 *            masks, no offsets; runs at level 6 only.
 */
typedef enum {
  AUTOFP_FMT_AUTOFP6 = 0,
  AUTOFP_FMT_AUTOFP6E = 1,
  AUTOFP_FMT_AUTOFP8 = 2,
  AUTOFP_FMT_FP6G = 3
} autofp_format;

/* Hyperparameters; autofp_default_params() fills the values of [AE] §5.1
 * ("Hyperparameters"). */
typedef struct {
  double  rho;             /* 0.2   weight refinement budget: floor(rho*k/4) refined subgroups */
  float   act_nmse_thresh; /* 0.003 activation subgroup NMSE threshold ([AE] §6.4)          */
  float   c2;              /* 2.0   AutoFP2 scale multiple c ([AE] App. B.4, Eq. 4)          */
  int32_t top_k;           /* 10    G_E top-K; top_k >= vocab means the whole vocabulary     */
  float   eps;             /* 1e-6  L_A stability term ([AE] Eq. 1; value not in the paper)  */
  double  tau;             /* 0.10  entropy threshold between decode regimes ([AE] §3.1)     */
  double  lambda_d;        /* 0.7   decode metric weight M = l*L_A + (1-l)*G_E (Table 1)     */
  int32_t alpha;           /* 4     trend lengths of Table 1 (alpha > beta)                  */
  int32_t beta;            /* 2                                                              */
  int32_t n_p;             /* 2     prefill trend length                                     */
  int32_t gemv_waves;      /* 0     autofp_gemv wavefronts per 16-row tile: 0 = automatic,   */
                           /*       or 1, 2, 4, 8, 16 to request it (tuning and tests); the  */
                           /*       kernel raises it to ceil(k / 4096) when that is larger   */
} autofp_params;

/*
 * Device-resident state of the runtime policy for one sequence (one batch
 * row). Zero-fill it before a sequence starts; autofp_policy_update() owns it
 * afterwards. mean/m2/count are the running (Welford) statistics of the
 * metric M in the current phase; up/down count consecutive layers above /
 * below the running mean; bits is the level chosen for the next layer.
 */
typedef struct {
  double  mean;
  double  m2;
  int32_t count;
  int32_t up;
  int32_t down;
  int32_t bits;
  int32_t spike;           /* prefill: the spike layer has been seen */
  int32_t reserved[3];
} autofp_policy_state;

/*
 * One AutoFP tensor ([AE] §4: "E2M1 base values with E4M3 group scales, signed
 * offsets d stored as one byte per refined subgroup, and refinement masks
 * stored as 4 bits per group along the K-dimension"; layout of Fig. 23).
 *
 *  codes        [rows][k/2]   E2M1 codes s|e1|e0|m, element 2i in the low nibble.
 *  scales       [rows][k/16]  E4M3 (OCP E4M3FN) group scales B.
 *  tensor_scale [1]           FP32 tensor scale T ([AE] Eq. 2).
 *  mask         WEIGHT:     [ceil(k/32)]        one 4-bit mask per group shared by
 *                                               all rows (M_W, [AE] §3.2);
 *               ACTIVATION: [rows][ceil(k/32)]  per-row mask M_A.
 *               Group 2g is the low nibble; bit s of a nibble = subgroup s.
 *               NULL when the tensor carries no 6-bit refinement.
 *  offsets      WEIGHT:     [rows][n_refined]   one byte per refined subgroup, in
 *                                               ascending (group, subgroup) order,
 *                                               followed by 16 bytes of padding that
 *                                               autofp_gemv may read (any content,
 *                                               never written);
 *               ACTIVATION: [rows][k/4]         one byte per subgroup (0 where the
 *                                               subgroup is not refined).
 *               Byte = four 2-bit two's-complement d, element e of the subgroup
 *               in bits [2e+1:2e]; value delta = d/8 ([AE] §3.2, fixed step).
 *  n_refined    WEIGHT only: number of refined subgroups per row (= popcount of
 *               mask); 0 otherwise.
 *  format       autofp_format (0 = AUTOFP6, the layout above). AUTOFP8 offsets
 *               take two bytes per subgroup (WEIGHT [rows][2 n_refined] + 16
 *               bytes of padding, ACTIVATION [rows][k/2]); FP6G codes are
 *               [rows][3k/4] and mask and offsets are NULL.
 */
typedef struct {
  int64_t  rows;
  int64_t  k;
  int32_t  kind;        /* autofp_kind */
  int32_t  n_refined;
  uint8_t *codes;
  uint8_t *scales;
  float   *tensor_scale;
  uint8_t *mask;
  uint8_t *offsets;
  int32_t  format;      /* autofp_format */
  int32_t  reserved;    /* 0 */
} autofp_packed;

/* Operations whose scratch space autofp_workspace_bytes() sizes. */
typedef enum {
  AUTOFP_OP_QUANTIZE = 0,     /* rows, k of the input                           */
  AUTOFP_OP_SELECT_MASK = 1,  /* rows, k of the weight                          */
  AUTOFP_OP_GEMV = 2,         /* rows = batch (tokens), k                       */
  AUTOFP_OP_GEMM = 3,         /* rows = tokens, k                               */
  AUTOFP_OP_SIGNALS = 4,      /* rows = batch, k = vocab (any vocab >= 1)       */
  AUTOFP_OP_KV_WRITE = 5,     /* rows = tokens * KV heads, k = head_dim         */
  AUTOFP_OP_KV_ATTENTION = 6, /* rows = batch * query heads, k = max_pages      */
  AUTOFP_OP_GPTQ = 7,         /* rows, k of the weight                          */
  AUTOFP_OP_EPILOGUE = 8      /* rows, k of the epilogue's output               */
} autofp_op;

/* Fills *p with the paper's hyperparameters. Errors: NULL. */
autofp_status autofp_default_params(autofp_params *p);

/* Human-readable name of a status code (static string, never NULL). */
const char *autofp_status_string(autofp_status s);

/* Bytes of each buffer of one packed tensor of format `format`, written to
 * out_bytes (host): [0] codes, [1] scales, [2] tensor_scale, [3] mask,
 * [4] offsets (for a WEIGHT: rows * n_refined * (2 for AUTOFP8, else 1) + 16,
 * the padding included). refine = 0 gives 0 for mask and offsets. For WEIGHT,
 * n_refined is the value autofp_weight_refined_count() returns.
 * Errors: NULL, SHAPE, KIND, ARG (format unknown, or FP6G with refine). */
autofp_status autofp_packed_bytes(int64_t rows, int64_t k, int32_t kind, int32_t format,
                                  int32_t refine, int32_t n_refined, size_t out_bytes[5]);

/* Number of refined subgroups per weight row: floor(rho * k / 4), at most two
 * per group ([AE] App. E, Alg. 1: budget rho*K/4, l_j in {0, 1, 2}).
 * Host only, no GPU work. Errors: NULL, SHAPE, ARG (rho outside [0, 1]). */
autofp_status autofp_weight_refined_count(int64_t k, const autofp_params *p, int32_t *n_refined);

/* Scratch bytes that operation `op` needs for a [rows x k] operand (host).
 * Errors: NULL, SHAPE, ARG. */
autofp_status autofp_workspace_bytes(int32_t op, int64_t rows, int64_t k, size_t *bytes);

/*
 * Weight mask M_W for a weight w [rows x k] (fp32, device), [AE] §3.2 and
 * App. E, Alg. 1 (budget allocation) with the identity Hessian:
 *  1. NVFP4-encode w (as autofp_quantize does) and, per row n, group j and
 *     subgroup s, the fp64 reduction in squared error from refining it:
 *       g = sum over the 4 elements of (eb*eb - er*er),
 *       eb = w - T*B*q, er = w - T*B*(q + delta),
 *     with d and delta those of `format` (AUTOFP6, AUTOFP6E or AUTOFP8; at
 *     level 8 for AUTOFP8);
 *  2. sum g over rows n = 0..rows-1 in that order (fp64);
 *  3. refine the top n_refined (group, subgroup) candidates, at most two per
 *     group, ordered by gain (descending), then group, then subgroup.
 * Writes mask_out [ceil(k/32)] (device). n_refined comes from
 * autofp_weight_refined_count(). Errors: NULL, SHAPE, ARG (also FP6G or an
 * unknown format), WORKSPACE, HIP.
 */
autofp_status autofp_select_weight_mask(const float *w, int64_t rows, int64_t k, int32_t format,
                                        const autofp_params *p, uint8_t *mask_out,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Encode x [out->rows x out->k] (x_dtype F32 or BF16; bf16 is widened exactly)
 * into AutoFP, [AE] App. B.1 Eqs. 2-3 (NVFP4 base), §3.2 (AutoFP6 offsets):
 *   T = amax(x) / 2688;  B_j = E4M3(amax(x_j) / (6T));  q_i = E2M1(x_i / (T B_j))
 * in fp32 with round-to-nearest-even (ties to even), E2M1 saturating at 6,
 * E4M3 at 448, canonical +0; T is one scalar over the whole call.
 *  - WEIGHT with out->mask != NULL: out->mask must already hold M_W (from
 *    autofp_select_weight_mask) and out->n_refined its popcount; writes the
 *    compacted offsets d = argmin over {-2,-1,0,+1} of |x/(TB) - q - d/8|
 *    (ties to the smaller |d|).
 *  - ACTIVATION with refine != 0: writes M_A - subgroups whose NMSE
 *    ((e0^2+e1^2)+e2^2)+e3^2 > thresh * ((v0^2+v1^2)+v2^2)+v3^2 (fp32, v = x/(TB),
 *    e = v - q; [AE] §6.4) that are not in exclude_mask (the layer's M_W,
 *    [ceil(k/32)], may be NULL) - and the dense offsets.
 *  - out->format selects the offsets (autofp_format): AUTOFP6E takes
 *    d = argmin |r - d 2^(e-3)|, AUTOFP8 d = argmin over {-8..7} of |r - d/8|
 *    (r = x/(TB) - q, ties to the smaller |d|); the masks follow the same
 *    rules. FP6G encodes T = amax/3360, B_j = E4M3(amax_j/(7.5 T)),
 *    q_i = E2M3(x_i/(T B_j)) (nearest, ties to the even code, saturating at
 *    7.5); it takes refine = 0 and no mask.
 * Errors: NULL, SHAPE, KIND, DTYPE, WORKSPACE, MISSING_REFINEMENT, ARG
 * (format unknown; FP6G with refine or a mask), HIP.
 */
autofp_status autofp_quantize(const void *x, int32_t x_dtype, int32_t refine,
                              const uint8_t *exclude_mask, const autofp_params *p,
                              autofp_packed *out, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Refinement-aware GPTQ calibration of a weight w [rows x k] (fp32, device):
 * [AE] App. E, Algorithm 1, with the group error of Eq. 7
 *   E_j(m) = sum_{i in J} H_ii ||W[:, i] - What[:, i](m)||^2
 * (J the 16 columns of group j, What(m) the group dequantized with the
 * refined values T B (q + d/8) on the subgroups of mask m):
 *  - T = amax(w) / 2688, fixed (line 4);
 *  - the budget floor(rho k / 4) is spread over the groups by the greedy of
 *    lines 5-12 on the original weights (at most two per group), which is
 *    the selection of autofp_select_weight_mask with each column's gain
 *    weighted by h_diag;
 *  - for each group j in order (lines 13-24): B, q and d from the
 *    error-compensated weights (rounded to fp32, encoded as autofp_quantize
 *    does); the group's mask m*_j = the l_j subgroups with the largest Eq. 7
 *    reductions over all rows (a tie goes to the lower subgroup); the group's
 *    codes, scale and offsets; its error r = W_J - What_J(m*_j) propagated
 *    to every later column: e U_JJ = r (forward substitution), then
 *    W[:, later] -= e U[J, later], in fp64 with each product and sum rounded
 *    in index order.
 * u [k x k] fp64 row-major: the upper Cholesky factor of the inverse of the
 * (dampened) Hessian, H^-1 = U^T U (entries below the diagonal are not read;
 * its diagonal must be positive); h_diag [k] fp64: the Hessian's diagonal
 * (H_ii >= 0). Writes out->codes, scales, tensor_scale, mask (M_W, popcount
 * n_refined) and offsets; out: WEIGHT, AUTOFP6, rows and k of w, mask and
 * offsets allocated, n_refined = autofp_weight_refined_count(k, p).
 * k <= 65536, rows <= 1048560. Workspace: autofp_workspace_bytes(
 * AUTOFP_OP_GPTQ, rows, k) (the fp64 working weights: 10 rows k bytes and
 * more). 4 launches per 16-column group.
 * Errors: NULL, SHAPE, KIND, ARG (format, n_refined, alignment), WORKSPACE,
 * MISSING_REFINEMENT, HIP.
 */
autofp_status autofp_gptq_quantize(const float *w, int64_t rows, int64_t k, const double *u,
                                   const double *h_diag, const autofp_params *p, autofp_packed *out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Elementwise step between a linear layer's output and the next layer's input
 * (autofp_epilogue_quantize). */
typedef enum {
  AUTOFP_EPI_COPY = 1,      /* v = z[:, :k]                                   */
  AUTOFP_EPI_RESIDUAL = 2,  /* v = residual + z[:, :k]                        */
  AUTOFP_EPI_SWIGLU = 3,    /* v = silu(z[:, :k]) * z[:, k:2k], silu(g) = g / (1 + e^-g) */
  AUTOFP_EPI_RESIDUAL_RMSNORM = 4  /* u = residual + z[:, :k]; v = u * c, per row
                                      c = 1 / sqrt(sum u^2 / k + 1e-5)  (RMSNorm, unit gain) */
} autofp_epilogue_op;

/*
 * Producer epilogue: the post-processing of a completed linear output into
 * the next layer's input activation ([AE] §6.4, "Shared Post-Processing
 * Unit": completed outputs are quantized into the next layer's activations,
 * with the NMSE refinement outside M_W and the non-linear operations). From
 * z [out->rows][ldz] fp32 (a linear layer's output, e.g. from autofp_gemv)
 * it forms v [out->rows][out->k] in fp32 with `op`, writes v to v_out (may be
 * NULL) and encodes v into `out` exactly as autofp_quantize would encode v
 * (same arguments refine / exclude_mask / p, same results bit for bit). One
 * launch for out->rows * roundup(out->k, 256) <= 32768, two above. COPY and
 * RESIDUAL need ldz >= k, SWIGLU ldz >= 2k; residual [rows][k] fp32 (RESIDUAL
 * and RESIDUAL_RMSNORM). z, residual, v_out 16-byte aligned, ldz % 4 == 0.
 * Workspace as autofp_quantize (AUTOFP_OP_QUANTIZE, rows, k); out->kind
 * ACTIVATION.
 * RESIDUAL_RMSNORM is a pre-norm block's residual add and the RMSNorm of the
 * next linear's input in one step: v_out (if not NULL) receives the residual
 * sum u (the new hidden state, fp32), and the normalized v is what gets
 * encoded. Per row the squares of u are summed in fp64 (each square exact) and
 * c = 1 / sqrt(sum / k + 1e-5) is rounded to fp32; v = u * c in fp32. Its
 * workspace is autofp_workspace_bytes(AUTOFP_OP_EPILOGUE, rows, k) (the
 * encode's plus one fp32 scale per row); one launch for the same small sizes,
 * four above (row scales, partial maxima, mask prefix, encode).
 * Errors: NULL, SHAPE, KIND, ARG, WORKSPACE, MISSING_REFINEMENT, HIP.
 */
autofp_status autofp_epilogue_quantize(int32_t op, const float *z, int64_t ldz, const float *residual,
                                       float *v_out, int32_t refine, const uint8_t *exclude_mask,
                                       const autofp_params *p, autofp_packed *out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * The last producer epilogue of a decoder layer together with the layer's
 * policy step ([AE] §6.4, the post-processing unit forming the next layer's
 * input; §3.1, Eq. 1 and Table 1, the runtime policy at the layer boundary):
 * autofp_epilogue_quantize(AUTOFP_EPI_RESIDUAL_RMSNORM, z, ldz, residual,
 * v_out, refine, exclude_mask, p, out, ...) followed by
 * autofp_policy_layer(phase, layer, new_sequence, h_prev, v_out, AUTOFP_F32,
 * out->k, g_e, out->rows, p, state, l_a_out, bits_rows, bits_layer, ...).
 * The same results: v_out (the new hidden state u = residual + z) and the
 * encoded bytes bit for bit; L_A per row from fp64 sums of the exact
 * differences and squares, equal to autofp_policy_layer's up to the order of
 * the fp64 additions; the levels, bits_layer and state as the Table 1 step
 * with that L_A. One launch for out->rows * roundup(out->k, 256) <= 32768; above,
 * the epilogue's launches and then the policy's.
 * z [rows][ldz], residual, v_out (required) and h_prev (the layer's input
 * hidden state) [rows][k], all fp32, 16-byte aligned; v_out must not overlap
 * z, residual or h_prev (equal pointers are rejected). The policy arguments
 * as autofp_policy_layer (g_e [rows] fp32, state [rows], l_a_out [rows] fp32,
 * bits_rows [rows] int32, bits_layer [1] or NULL). Workspace
 * autofp_workspace_bytes(AUTOFP_OP_EPILOGUE, rows, k).
 * Errors: NULL, SHAPE, KIND, ARG, WORKSPACE, MISSING_REFINEMENT, HIP.
 */
autofp_status autofp_layer_epilogue(const float *z, int64_t ldz, const float *residual, float *v_out,
                                    const float *h_prev, int32_t refine, const uint8_t *exclude_mask,
                                    int32_t phase, int32_t layer, int32_t new_sequence, const float *g_e,
                                    const autofp_params *p, autofp_policy_state *state, float *l_a_out,
                                    int32_t *bits_rows, int32_t *bits_layer, autofp_packed *out,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * autofp_quantize for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, checks and results, but no workspace argument. Its scratch
 * (the amax partials and the weight-mask prefix table) lives in a static
 * 64 KiB device array of the library, one per GPU, held until the process
 * ends; nothing is allocated. Sizes whose scratch would exceed 64 KiB are
 * rejected with AUTOFP_ERR_WORKSPACE: that is any k above 491488 (rows are
 * not limited). Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (different streams, different host threads)
 * race and must be serialized by the caller.
 * Errors: those of autofp_quantize (WORKSPACE for k > 491488); HIP also when
 * the array's device address cannot be obtained.
 */
autofp_status autofp_quantize_noalloc(const void *x, int32_t x_dtype, int32_t refine,
                                      const uint8_t *exclude_mask, const autofp_params *p,
                                      autofp_packed *out, void *stream);

/*
 * Decode-phase linear layer ([AE] §3.1-3.2, §4): for b < x->rows, n < w->rows
 *   y[b][n] = sum_k What[n][k] * Xhat[b][k]
 * with the operands at precision level `bits`:
 *   2: W as AutoFP2 digits c*T*B*Q, X as NVFP4 (W2A4);
 *   4: both NVFP4 T*B*q;
 *   6: W refined on M_W, X refined on M_A: T*B*(q + d/8) (W6A6).
 * Products are exact and accumulated in fp32. y is [x->rows x w->rows]
 * row-major, y_dtype F32 or BF16 (round to nearest even).
 * If bits_dev != NULL the level is read on the device when the kernels run
 * (graph-capturable, no host read); `bits` is then ignored but a level-6 call
 * must be allowed by the operands (both carry refinement).
 * Best for x->rows <= 64; larger batches run in slices of 64 tokens. k must
 * be at most 2^22 (4194304); with at most 16 tokens, a level-6 call (or one
 * with bits_dev) needs k <= 65536. Any number of tokens: the kernels address
 * the activations one tile of rows at a time.
 * Formats (autofp_format): w and x must have the same format. AUTOFP6E and
 * AUTOFP8 run levels 2 and 4 as AUTOFP6 (their NVFP4 base), level 6 with
 * their own delta, and AUTOFP8 also level 8: T*B*(q + d/8) with the full
 * 4-bit d on both operands (W8A8). FP6G runs level 6 only, without bits_dev:
 * T*B*q with its E2M3 codes (W6A6 of the comparator). Levels above 4 of the
 * variant formats (and any bits_dev call on them) need k % 64 == 0 and run
 * on the prefill GEMM's tiles.
 * Errors: NULL, SHAPE, KIND, BITS, MISSING_REFINEMENT, DTYPE, WORKSPACE, ARG
 * (formats differ or unknown), HIP.
 */
autofp_status autofp_gemv(const autofp_packed *w, const autofp_packed *x, int32_t bits,
                          const int32_t *bits_dev, void *y, int32_t y_dtype,
                          const autofp_params *p, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Decode-phase linear layer for a batch whose rows (tokens) run at different
 * precision levels ([AE] §4.2 "Serving Mixed-Precision Batches": requests of
 * one batch that chose different levels share one GEMM over the union of
 * their refinements, Fig. 6; the levels come from the policy per request,
 * §3.1 and autofp_policy_update's bits_rows):
 *   y[b][n] = sum_k What_l[n][k] * Xhat_l[b][k],  l = bits_rows[b] in {2, 4, 6}
 * with the operands of level l as in autofp_gemv (row b at level 6 uses its
 * own activation refinement M_A and the weight refinement M_W; at 4 plain
 * NVFP4; at 2 the AutoFP2 weight digits times the NVFP4 activation). Each row
 * equals the row autofp_gemv gives at that row's level. bits_rows [x->rows]
 * int32 (device, read when the kernels run); a value outside {2, 4, 6} gives
 * a zero row. Any row may be at level 6, so both operands must carry their
 * refinement (weight mask and offsets; activation mask and offsets).
 * k % 128 == 0 and k <= 2^22; any number of rows (slices of 64). Workspace as
 * autofp_gemv. Both operands AUTOFP6 (format 0). Errors: NULL, SHAPE, KIND,
 * MISSING_REFINEMENT, DTYPE, WORKSPACE, ARG (also another format), HIP.
 */
autofp_status autofp_gemv_rows(const autofp_packed *w, const autofp_packed *x, const int32_t *bits_rows,
                               void *y, int32_t y_dtype, const autofp_params *p, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Prefill-phase linear layer ([AE] §4.1, "Extended-K GEMM": the same product
 * as the decode GEMV, run for every prompt token at once; §5.3 prefill of 1K
 * to 128K input tokens): y = Xhat . What^T for any number of tokens, tiled
 * for the matrix cores (256-token x 256-row tiles when K % 64 == 0). The
 * fp16 activations are staged in the workspace (autofp_workspace_bytes(
 * AUTOFP_OP_GEMM, tokens, k): 2 * tokens * round_up(k, 256) bytes plus the
 * weight-mask prefix). k <= 2^22. Same arguments, results, formats and
 * errors as autofp_gemv.
 */
autofp_status autofp_gemm(const autofp_packed *w, const autofp_packed *x, int32_t bits,
                          const int32_t *bits_dev, void *y, int32_t y_dtype,
                          const autofp_params *p, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * The two runtime-policy signals ([AE] §3.1):
 *  - entropy_out[b] = G_E of logits row b: softmax over the top_k largest
 *    logits, H = -sum p ln p, divided by ln(top_k) (ln(vocab) when
 *    top_k >= vocab). logits [batch x vocab] fp32. top_k must be 1..32 or
 *    >= vocab. Masked entries may hold -inf (probability 0, no term of H) as
 *    long as each row has at least one finite logit.
 *  - update_out[b] = L_A = ||h_cur[b] - h_prev[b]||_2 / (||h_prev[b]||_2 + eps)
 *    ([AE] Eq. 1); h_prev, h_cur [batch x hidden] in h_dtype (F32 or BF16).
 * Either signal is skipped when its output pointer is NULL (its inputs may
 * then be NULL too). G_E needs a workspace of autofp_workspace_bytes(
 * AUTOFP_OP_SIGNALS, batch, vocab) bytes (per-slice candidates of the
 * vocabulary); L_A needs none (workspace may be NULL when entropy_out is).
 * Errors: NULL, SHAPE, DTYPE, ARG, WORKSPACE, HIP.
 */
autofp_status autofp_policy_signals(const float *logits, int64_t batch, int64_t vocab,
                                    const void *h_prev, const void *h_cur, int32_t h_dtype,
                                    int64_t hidden, const autofp_params *p,
                                    float *entropy_out, float *update_out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * One step of the runtime precision policy after layer `layer` has run
 * ([AE] §3.1 and Table 1), for every batch row b, on the device:
 *   prefill (phase 0): M = L_A; layers up to and including the first spike
 *     (M > mu + 3 sigma with at least two earlier values) run at 6 bits;
 *     after it, n_p consecutive layers below (above) mu lower (raise) the next
 *     layer one level of {2, 4, 6}, saturating.
 *   decode (phase 1): M = lambda_d * L_A + (1 - lambda_d) * G_E, G_E of the
 *     previous step (g_e[b]); layer 0 runs at 4 bits; with G_E >= tau, beta
 *     consecutive layers above mu raise and alpha below lower the next layer;
 *     with G_E < tau, alpha and beta swap.
 * mu and sigma (population) are running statistics of the earlier M of the
 * sequence in the current phase, excluding the value being judged. At
 * layer 0 the trend counters restart and the level is reset (6 in prefill,
 * 4 in decode); new_sequence != 0 also clears the statistics.
 * l_a [batch] fp32 (device): L_A of this layer; g_e [batch] fp32 (device,
 * decode only, may be NULL in prefill); state [batch] (device);
 * bits_rows [batch] int32 (device, out): level of layer+1 per row;
 * bits_layer [1] int32 (device, out, may be NULL): the highest level over the
 * rows, the level at which a batched layer runs.
 * Errors: NULL, SHAPE, ARG (phase not 0/1, layer < 0), HIP.
 */
autofp_status autofp_policy_update(int32_t phase, int32_t layer, int32_t new_sequence,
                                   const float *l_a, const float *g_e, int64_t batch,
                                   const autofp_params *p, autofp_policy_state *state,
                                   int32_t *bits_rows, int32_t *bits_layer, void *stream);

/*
 * The per-layer step of the policy in one call ([AE] §3.1: Eq. 1, then
 * Table 1): L_A of every row from the layer's input and output hidden states,
 * written to l_a_out [batch] fp32 (device), then autofp_policy_update with it.
 * The results equal autofp_policy_signals (update part) followed by
 * autofp_policy_update, value for value (the same fp64 summation order). Up to
 * 4 rows it is one launch; above, the two launches. h_prev, h_cur
 * [batch][hidden] in h_dtype (F32 or BF16); other arguments as in
 * autofp_policy_update.
 * Errors: NULL, SHAPE, DTYPE, ARG, HIP.
 */
autofp_status autofp_policy_layer(int32_t phase, int32_t layer, int32_t new_sequence,
                                  const void *h_prev, const void *h_cur, int32_t h_dtype,
                                  int64_t hidden, const float *g_e, int64_t batch,
                                  const autofp_params *p, autofp_policy_state *state,
                                  float *l_a_out, int32_t *bits_rows, int32_t *bits_layer,
                                  void *stream);

/*
 * ---------------------------------------------------------------------------
 * AutoFP KV cache and decode attention ([AE] §4.1, last paragraph; §5.1)
 * ---------------------------------------------------------------------------
 * K and V are kept in AutoFP in two page types of equal byte size ([AE] §4.1):
 * a base page holds 64 tokens (the KV page size T of [AE] §5.1) with their
 * NVFP4 base values; a refinement page holds 32 refined tokens with base
 * values and signed offsets, the offsets stored as 4*delta = d/2 in E2M1
 * ({-1, -0.5, 0, +0.5}). Every (token, KV head) vector of head_dim = 128
 * elements is one NVFP4 row: E4M3 scale per 16 elements along the head
 * dimension, one FP32 tensor scale for the whole K cache and one for V. A
 * refined token has an offset d for every subgroup (the argmin of autofp_quantize).
 *
 * Pools: k_pages and v_pages are [n_pages][h_kv][AUTOFP_KV_PAGE_BYTES]; one
 * page id addresses the same tokens in both pools and in every KV head; its
 * type is page_kind[id] (0 base, 1 refinement). Layout of one KV-head section
 * (C = 64 tokens for a base page, 32 for a refinement page; token t of the page;
 * E2M1 nibbles with element 2i in the low nibble):
 *   K: codes   [C][64]  at 0          token-major, dims in order
 *      scales  [C][8]   at 64*C       E4M3, group j of token t at 8*t + j
 *      offsets [C][64]  at 72*C       (refinement pages) E2M1 codes of d/2, like codes
 *   V: codes   [C/8][16][8][4] at 0   block (t/8, dim/8), then dim%8: one dword per
 *                                     dim holds tokens 8*(t/8) .. +7, token t in nibble t%8
 *      scales  [8][C]   at 64*C       group-major: group j of token t at C*j + t
 *      offsets (refinement pages) at 72*C, laid out like the V codes
 * A refinement section uses 4352 of its 4608 bytes; the tail is never read.
 *
 * A sequence b owns the pages page_table[b][0 .. seq_pages[b]-1] (any order:
 * the attention of one query does not depend on the order of the context);
 * page id p holds page_tokens[p] tokens in positions 0 .. page_tokens[p]-1
 * (clamped to its capacity), so a sequence may keep one partly filled page of
 * each type. Page ids outside [0, n_pages) are skipped as empty.
 */
#define AUTOFP_KV_PAGE_TOKENS 64     /* base-page capacity ([AE] §5.1, T = 64)  */
#define AUTOFP_KV_HEAD_DIM 128       /* the head dimension the kernels support  */
#define AUTOFP_KV_PAGE_BYTES 4608    /* one KV head of one page: 64 x (64 + 8)  */

typedef struct {
  int32_t  h_kv;                   /* KV heads                                      */
  int32_t  head_dim;               /* must be AUTOFP_KV_HEAD_DIM                    */
  int32_t  n_pages;                /* pages in each pool                            */
  int32_t  max_pages;              /* columns of page_table                         */
  uint8_t *k_pages;                /* [n_pages][h_kv][AUTOFP_KV_PAGE_BYTES]         */
  uint8_t *v_pages;                /* [n_pages][h_kv][AUTOFP_KV_PAGE_BYTES]         */
  const uint8_t *page_kind;        /* [n_pages] 0 base, 1 refinement                */
  float   *k_scale;                /* [1] FP32 tensor scale T of the K cache        */
  float   *v_scale;                /* [1] FP32 tensor scale T of the V cache        */
  const int32_t *page_table;       /* [batch][max_pages] page ids of each sequence  */
  const int32_t *seq_pages;        /* [batch] pages in use (clamped to max_pages)   */
  const int32_t *page_tokens;      /* [n_pages] tokens held by each page            */
} autofp_kv_cache;

/*
 * Encode new K/V tokens into their pages. k and v are [n_tokens][h_kv][128]
 * in `dtype` (F32 or BF16, bf16 widened exactly); slots [n_tokens] (device)
 * give each token's destination as page_id * 64 + position, with position
 * below the page's capacity (64 base, 32 refinement); other slots are skipped.
 * set_scale != 0: first sets *k_scale = amax(k) / 2688 and *v_scale =
 * amax(v) / 2688 over this call's tokens ([AE] App. B.1, Eq. 2), as for a
 * prompt; otherwise the stored tensor scales are used and values beyond
 * 6 * 448 * T saturate. The tensor scales are shared by every page of the
 * cache and read by autofp_kv_attention for all of them: set them only when
 * the cache is first filled (its first prompt). A later call with
 * set_scale != 0 rescales the pages already written by other calls, which then
 * decode wrongly; later prompts and decode tokens use set_scale = 0. Group scales and codes follow autofp_quantize (Eqs.
 * 2-3, fp32, ties to even); tokens of refinement pages also get their offsets.
 * The page table fields of `cache` are not read. Workspace:
 * autofp_workspace_bytes(AUTOFP_OP_KV_WRITE, n_tokens * h_kv, 128) bytes
 * (may be NULL when set_scale == 0).
 * Errors: NULL, SHAPE, DTYPE, WORKSPACE, ARG, HIP.
 */
autofp_status autofp_kv_write(const void *k, const void *v, int32_t dtype, int64_t n_tokens,
                              const int32_t *slots, int32_t set_scale,
                              const autofp_kv_cache *cache, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Decode attention over an AutoFP KV cache ([AE] §4.1): for batch row b and
 * query head h (KV head g = h / (h_q / h_kv)),
 *   s_j = sm_scale * q[b][h] . K_hat[g][j],  p = softmax(s) over the
 *   sequence's tokens,  out[b][h] = sum_j p_j V_hat[g][j]
 * with K_hat, V_hat = T * B * q (NVFP4) and, at level 6, T * B * (q + d/8) for
 * tokens of refinement pages. Levels 2 and 4 read the KV cache at 4 bits (the
 * 2-bit level is for weights only, [AE] §3.1 W2A4KV4). bits_dev != NULL: the
 * level is read on the device at run time (`bits` ignored).
 * q [batch][h_q][128] F32 or BF16. On the matrix cores K_hat and V_hat are
 * exact in fp16, and the query and the probabilities enter as sums of two
 * fp16 parts (relative error about 2^-22); products accumulate in fp32.
 * out [batch][h_q][128] fp32. h_q must be a multiple of h_kv with at
 * most 16 query heads per KV head. A sequence with no tokens gives zeros.
 * Workspace: autofp_workspace_bytes(AUTOFP_OP_KV_ATTENTION, batch * h_q,
 * cache->max_pages) bytes (partial results of the context splits).
 * Errors: NULL, SHAPE, BITS, DTYPE, WORKSPACE, ARG, HIP.
 */
autofp_status autofp_kv_attention(const void *q, int32_t q_dtype, int64_t batch, int32_t h_q,
                                  const autofp_kv_cache *cache, int32_t bits,
                                  const int32_t *bits_dev, float sm_scale, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AUTOFP_H */
