/*
 * quads.h -- C ABI of libquads, the gfx950 (MI355X) implementation of the
 * QUADS rollout/trainer hot path: NVFP4 activation quantization, Residual
 * Activation Compensation (RAC), the W4A4+RAC grouped expert GEMM, and the
 * trainer-side weight quantize-dequantize (QDQ).
 *
 * Method sources (three web pages about the paper "QUADS: Stabilizing NVFP4
 * Reinforcement Learning for MoE via QUantization-error Alignment across Dual
 * Sides"):
 *   [Gist]  gist.science "Technische Samenvatting: QUADS" -- section 1
 *           (NVFP4 W4A4 GEMMs; the E2M1 grid has eight levels per sign),
 *           section 2.1 (activations are re-quantized online on every
 *           forward; weights are aligned by sharing one QDQ path),
 *           section 2.2-A (asymmetric W4A16 QAT: NVFP4 fake-quantized
 *           weights, BF16 activations), section 2.2-B (RAC: a binary mask of
 *           the top k% channels by residual magnitude, a second-pass
 *           quantization of their residual, added to the quantized path).
 *   [Wiki]  AI-Wiki summary, "Methodology" (the compensation is added before
 *           the native W4A4 GEMM).
 *
 * NVFP4 encoding used throughout (the pages name the format, not its
 * layout): 16-element blocks along the last (contraction) axis; one OCP FP8
 * E4M3 block scale per block (no infinities, max 448, never NaN here); one
 * FP32 scale g per tensor, decode direction (value = e2m1 * e4m3 * g);
 * rounding is nearest-even with saturation; g = fl32(amax / 2688), or 1 for
 * an all-zero tensor; block scale s = E4M3(fl32(fl32(amax_block / 6) / g));
 * element code = sign << 3 | nearest E2M1 magnitude of fl32(|x| / fl32(dec(s) * g))
 * (the sign bit is kept for zeros).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller (e.g. from
 *     torch.empty on the GPU).  The library never allocates device memory;
 *     scratch space is a caller-provided workspace whose size is returned by
 *     the matching *_workspace_bytes() query.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; they never synchronize the host.
 *   - Layouts are row-major.  Packed codes: [rows, cols/2] bytes, element 2j
 *     in the low nibble of byte j.  Block scales: [rows, cols/16] bytes.
 *   - Return value: QUADS_OK or a negative quads_status_t; on error nothing is
 *     enqueued and quads_last_error() (thread-local) describes the problem.
 *     Nothing throws or aborts across the ABI.
 *   - Array pointers must be 16-byte aligned (QUADS_ERR_ARG otherwise); fresh
 *     torch allocations are.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified (but memory-safe)
 *     results.
 */
#ifndef QUADS_H
#define QUADS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QUADS_OK = 0,
  QUADS_ERR_ARG = -1,       /* null pointer, bad enum, k outside [0,100] */
  QUADS_ERR_SHAPE = -2,     /* cols % 16 != 0, size overflow, unsupported shape */
  QUADS_ERR_WORKSPACE = -3, /* workspace missing or too small */
  QUADS_ERR_DEVICE = -4     /* HIP launch error (message in quads_last_error) */
} quads_status_t;

typedef enum { QUADS_F32 = 0, QUADS_BF16 = 1 } quads_dtype_t;

/* quads_quantize_nvfp4 flags */
#define QUADS_GSCALE_GIVEN 1u /* use out.gscale[b] as the tensor scale instead of computing it */
#define QUADS_WANT_SCORES 2u  /* also compute RAC channel scores (batch must be 1) */

/* An NVFP4 tensor of `batch` matrices of [rows, cols] (cols % 16 == 0). */
typedef struct {
  uint8_t *codes;  /* [batch, rows, cols/2] */
  uint8_t *scales; /* [batch, rows, cols/16] E4M3 */
  float *gscale;   /* [batch] FP32 tensor scales */
  int64_t batch, rows, cols;
} quads_nvfp4_t;

/* Thread-local description of the last error ("" if none). */
const char *quads_last_error(void);

/* Library version string. */
const char *quads_version(void);

/* ---------------------------------------------------------------------------
 * RAC sizes.  [Gist 2.2-B]: the mask keeps the top k% of channels.  nsel =
 * floor(cols * k / 100) in integer arithmetic; the selected-channel list is
 * padded to kpad = nsel rounded up to a multiple of 16 with index 0 and zero
 * residual.  Return -1 for invalid arguments (cols < 0, k outside [0,100]).
 * ------------------------------------------------------------------------- */
int64_t quads_rac_nsel(int64_t cols, int32_t k_percent);
int64_t quads_rac_kpad(int64_t nsel);

/* ---------------------------------------------------------------------------
 * quads_quantize_nvfp4 -- NVFP4-quantize x ([batch, rows, cols], F32 or BF16,
 * contiguous) into `out` (same batch/rows/cols).  Each of the `batch`
 * matrices gets its own tensor scale (one per weight matrix; batch = 1 for an
 * activation).  This is the online activation quantization of [Gist 2.1] and
 * the weight quantization shared by trainer and rollout.
 *
 * With QUADS_WANT_SCORES (batch == 1) it also writes the RAC channel scores
 * scores[c] = max over rows of |x - dequant(Q(x))| (FP32, [cols]), the
 * residual magnitudes [Gist 2.2-B] ranks channels by.
 *
 * ws: device workspace of at least quads_quantize_workspace_bytes(batch,
 * rows, cols) bytes (cross-workgroup amax partials).
 *
 * rows == 0: x, codes, scales and ws are neither read nor written (they may be
 * NULL); the largest of no magnitudes is taken as 0, so gscale[b] = 1 (unless
 * QUADS_GSCALE_GIVEN) and, with QUADS_WANT_SCORES, every score is 0.
 * ------------------------------------------------------------------------- */
size_t quads_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t cols);
quads_status_t quads_quantize_nvfp4(const void *x, quads_dtype_t dt, quads_nvfp4_t out,
                                    uint32_t flags, float *scores, void *ws, size_t ws_bytes,
                                    void *stream);

/* quads_quantize_nvfp4_noalloc -- quads_quantize_nvfp4 for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): no workspace argument; the amax
 * partials live in a fixed 1 MiB scratch array inside the library, one copy
 * per GPU, held until the process ends.  The caller still passes x, out and
 * scores.  The call allocates nothing and calls no allocating routine.
 * Limit: batch * P * 4 bytes <= 1 MiB, with P = min(1024, max(1,
 * ceil(rows * cols / 16384))) partials per matrix (e.g. up to 256 matrices
 * of at least 16 M elements, or 2048 matrices of at most 2 M elements);
 * larger calls return QUADS_ERR_WORKSPACE before anything is enqueued.
 * With QUADS_GSCALE_GIVEN no scratch is used.  The scratch of the calling
 * thread's current device is used, so `stream` must belong to that device.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from different threads) race; calls ordered
 * on one stream do not.  Results are identical to quads_quantize_nvfp4's. */
quads_status_t quads_quantize_nvfp4_noalloc(const void *x, quads_dtype_t dt, quads_nvfp4_t out,
                                            uint32_t flags, float *scores, void *stream);

/* ---------------------------------------------------------------------------
 * quads_rac_select -- RAC channel mask and second-pass residual quantization
 * [Gist 2.2-B].
 *   1. Rank channels by (scores desc, index asc); keep the first nsel =
 *      quads_rac_nsel(cols, k_percent); write them ASCENDING to sel_idx
 *      ([kpad] int32, pad entries 0).
 *   2. Residual G[r, j] = x[r, sel_j] - dequant(xq)[r, sel_j] (FP32, exact
 *      recomputation from x and xq), 0 for pad columns; quantize G to NVFP4
 *      into `res` ([rows, kpad], batch 1) with its own tensor scale, whose
 *      amax is the largest selected score.
 * x / dt: the activation that produced xq (batch 1); scores from
 * quads_quantize_nvfp4(QUADS_WANT_SCORES).  res.cols must equal kpad; with
 * k such that kpad == 0 only res.gscale[0] = 1 is written.  With rows == 0
 * the mask still comes from the scores (all 0 for an empty activation:
 * sel_idx = 0 .. nsel-1, res.gscale[0] = 1) and no row is touched.
 * Channel count limit: cols <= 16384 (larger shapes return QUADS_ERR_SHAPE
 * before anything is enqueued).  Two kernels are enqueued on `stream`: the
 * mask (one workgroup), then the rows; calls of bf16 rows with cols <= 2048
 * and at most one workgroup per CU (or many row groups per workgroup)
 * enqueue one kernel in which every workgroup finds the mask itself.
 * ------------------------------------------------------------------------- */
size_t quads_rac_select_workspace_bytes(int64_t rows, int64_t cols);
quads_status_t quads_rac_select(const void *x, quads_dtype_t dt, const quads_nvfp4_t *xq,
                                const float *scores, int32_t k_percent, int32_t *sel_idx,
                                quads_nvfp4_t res, void *ws, size_t ws_bytes, void *stream);

/* quads_rac_select_merged -- quads_rac_select that also writes the corrected
 * activation as one fp16 operand [Gist 2.2-B: the correction is added to the
 * quantized activation before the GEMM], merged_f16 [rows, cols] (device,
 * 16-byte aligned, caller-owned), in units of xq's tensor scale g_x:
 *   merged[r, c] = fp16( X'[r, c] + fl32(R'[r, j] * fl32(g_r / g_x)) )  for c = sel_j,
 *   merged[r, c] = X'[r, c]                                              otherwise,
 * with X' and R' the exact e2m1 * e4m3 values of xq and res (no tensor scale)
 * and one fp32 addition before the rounding.  Passing it to
 * quads_moe_w4a4_gemm (x_merged) lets the GEMM contract over K alone with no
 * merge pass of its own.  With kpad == 0 nothing is written (there is no
 * correction; the GEMM then takes the plain path); with rows == 0
 * merged_f16 may be NULL. */
quads_status_t quads_rac_select_merged(const void *x, quads_dtype_t dt, const quads_nvfp4_t *xq,
                                       const float *scores, int32_t k_percent, int32_t *sel_idx,
                                       quads_nvfp4_t res, void *merged_f16, void *ws, size_t ws_bytes,
                                       void *stream);

/* ---------------------------------------------------------------------------
 * quads_moe_w4a4_gemm -- token-permuted grouped expert GEMM with the RAC
 * segment (extended K), on fp16 MFMA with exact NVFP4 -> fp16 operand decode:
 *
 *   Y[i, n] = gw[e, seg(n)] * ( gx * sum_k W[e,n,k] X[t(i),k]
 *                             + gr * sum_j W[e,n,sel_j] R[t(i),j] )
 *
 * for routed row i of expert e (expert_offsets[e] <= i < expert_offsets[e+1]),
 * t(i) = row_token[i] (or i when row_token is NULL), W/X/R the e2m1 * e4m3
 * block values.  This is the quantized path plus the RAC correction, which
 * [Wiki Methodology] adds before the W4A4 GEMM and [Gist 2.2-B] adds to the
 * quantized output: the same sum.  With r_codes == NULL (or kpad == 0) it is
 * plain W4A4.
 *
 * Form of the RAC correction (quads_moe_gemm_args.rac_form; both stay within
 * max|Y - Y_exact| <= 1e-3 max|Y_exact| on the seeded workloads):
 *   QUADS_RAC_FORM_EXACT   the correction is an extended contraction over
 *                          the gathered weight columns: the GEMM accumulates
 *                          exact operand values in FP32 (accumulation
 *                          rounding only).  x_merged must be NULL.
 *   QUADS_RAC_FORM_MERGED  the correction is added to the activation before
 *                          the GEMM, as one fp16 operand per element
 *                          X' + fl32(R' * fl32(gr/gx)) in units of gx (the
 *                          quads_rac_select_merged definition; built by the
 *                          prepare step unless x_merged is given), so each
 *                          corrected element is rounded once more (relative
 *                          2^-11), and the GEMM contracts over K alone.
 *                          The prepare step's merge holds a row of K floats
 *                          and the mask on chip: 4*kpad + 4*K + K/8 <=
 *                          163584 bytes (any K <= 16384), else
 *                          QUADS_ERR_SHAPE (AUTO then takes EXACT).
 *   QUADS_RAC_FORM_AUTO    (0, the default) MERGED when x_merged is given,
 *                          for few rows per expert (num_rows <= 32 *
 *                          num_experts with K % 256 == 0, K <= 16384 and
 *                          N % 128 == 0: the decode shape) and where the
 *                          tile choice gives 256 x 256 tiles (large grouped
 *                          shapes); EXACT otherwise.  The choice depends
 *                          only on the arguments, so prepare and main agree.
 *
 * operand_mode QUADS_OPERANDS_BF16 is the trainer's W4A16 forward [Gist
 * 2.2-A]: x_bf16 [act_rows, K] times w_bf16 [E, N, K] (QDQ'd weights),
 * no scales, no residual.
 *
 * operand_mode QUADS_OPERANDS_BF16_QDQ is the same forward with the weight
 * QDQ fused in [Gist 2.2-A: every forward sees the discretized weights]:
 * w_bf16 holds the bf16 MASTER weights and w_gscale [E * n_seg] their tensor
 * scales (quads_weight_qdq with QUADS_SCALES_ONLY, one per (expert,
 * segment) matrix); each weight block is quantized to NVFP4 and dequantized
 * to bf16 in registers on its way to the matrix cores, with exactly the
 * operations of quads_weight_qdq (QUADS_GSCALE_GIVEN), so the product equals
 * quads_weight_qdq followed by QUADS_OPERANDS_BF16 bit for bit (same tile
 * schedule) while W_qdq is never written to memory.  K % 16 == 0; SWIGLU
 * needs n_seg == 2 (gate and up matrices with their own scales).
 *
 * operand_mode QUADS_OPERANDS_BF16_W4 is the same forward from the masters'
 * NVFP4 encoding: w_codes / w_scales / w_gscale hold the masters quantized
 * by quads_quantize_nvfp4 (one tensor scale per (expert, segment) matrix --
 * the codes quads_weight_qdq exports, and the trainer-to-rollout weight-sync
 * payload); each weight is decoded on its way to the matrix cores to its QDQ
 * value bf16(fl32(e2m1 * fl32(dec(s) * g))), so the product again equals
 * quads_weight_qdq followed by QUADS_OPERANDS_BF16 bit for bit, the GEMM
 * reads 0.5625 instead of 2 bytes per weight and W_qdq is never written.
 *
 * Epilogues: QUADS_EPI_NONE writes y [num_rows, N] (F32 or BF16);
 * QUADS_EPI_SWIGLU (n_seg must be 2: W rows [0, N/2) are the gate, [N/2, N)
 * the up projection) writes h [num_rows, N/2] BF16 with
 * h = silu(Y_gate) * Y_up.
 *
 * Shapes: K % 16 == 0, N % 128 == 0, num_experts in [1, 1024].  W4A4 calls
 * whose activation operand (codes, or the merged fp16 operand: act_rows x K)
 * or one expert's weight codes reach 4 GiB additionally need K % 128 == 0
 * and kpad % 64 == 0 (else QUADS_ERR_SHAPE): the register-staged kernels
 * address those tensors with 32-bit offsets.  expert_offsets is a DEVICE array of num_experts + 1
 * non-decreasing int32 with expert_offsets[0] = 0 and
 * expert_offsets[E] = num_rows (not checked on the host: reading it would
 * synchronize).  num_rows == 0: y and the activation operands may be NULL
 * and no row is written; y_gscale, if given, receives 1 (the tensor scale
 * of an empty output).
 * ws: at least quads_moe_gemm_workspace_bytes(args) bytes.
 * ------------------------------------------------------------------------- */
#define QUADS_OPERANDS_W4A4 0
#define QUADS_OPERANDS_BF16 1
#define QUADS_OPERANDS_BF16_QDQ 2
#define QUADS_OPERANDS_BF16_W4 3
#define QUADS_EPI_NONE 0
#define QUADS_EPI_SWIGLU 1

/* quads_moe_gemm_args.rac_form */
#define QUADS_RAC_FORM_AUTO 0
#define QUADS_RAC_FORM_EXACT 1
#define QUADS_RAC_FORM_MERGED 2

/* quads_moe_gemm_args.flags */
#define QUADS_GEMM_PREPARED 1u /* workspace already filled by quads_moe_gemm_prepare for
                                  these args: launch only the main GEMM kernel */

typedef struct {
  uint32_t struct_size;  /* sizeof(quads_moe_gemm_args) (ABI versioning) */
  uint32_t flags;        /* 0 or QUADS_GEMM_PREPARED */
  int32_t operand_mode;  /* QUADS_OPERANDS_W4A4 | QUADS_OPERANDS_BF16 */
  int32_t epilogue;      /* QUADS_EPI_NONE | QUADS_EPI_SWIGLU */
  int32_t y_dtype;       /* QUADS_F32 | QUADS_BF16 (EPI_NONE); SWIGLU writes BF16 */
  int32_t num_experts;   /* E */
  int32_t n_seg;         /* weight tensor scales per expert along N (1 or 2) */
  int64_t num_rows;      /* R: routed rows = output rows */
  int64_t act_rows;      /* rows of the activation tensors */
  int64_t N, K;
  /* W4A4 activation operand: codes [act_rows, K/2], scales [act_rows, K/16], gscale [1] */
  const uint8_t *x_codes;
  const uint8_t *x_scales;
  const float *x_gscale;
  /* RAC residual (NULL r_codes => plain W4A4): codes [act_rows, kpad/2],
     scales [act_rows, kpad/16], gscale [1], sel_idx [kpad] ascending */
  const uint8_t *r_codes;
  const uint8_t *r_scales;
  const float *r_gscale;
  const int32_t *sel_idx;
  int64_t kpad;
  /* W4A4 weights: codes [E, N, K/2], scales [E, N, K/16], gscale [E * n_seg]
     (BF16_QDQ: w_gscale only, the masters' tensor scales) */
  const uint8_t *w_codes;
  const uint8_t *w_scales;
  const float *w_gscale;
  /* BF16 operands (operand_mode QUADS_OPERANDS_BF16 or _BF16_QDQ) */
  const void *x_bf16; /* [act_rows, K] */
  const void *w_bf16; /* [E, N, K]: QDQ'd weights (BF16) or masters (BF16_QDQ) */
  const int32_t *row_token;      /* [num_rows] or NULL (identity) */
  const int32_t *expert_offsets; /* [E + 1], device */
  void *y;
  void *ws;
  size_t ws_bytes;
  /* Optional [act_rows, K] fp16 RAC-merged activation from
     quads_rac_select_merged (units of x_gscale), or NULL.  With a residual
     present the GEMM then contracts it over K alone (the merged form above),
     whatever the shape, and builds no merged operand of its own. */
  const void *x_merged;
  int32_t rac_form; /* QUADS_RAC_FORM_AUTO | _EXACT | _MERGED (see above) */
  /* Optional [1] float, device: the NVFP4 tensor scale of the bf16 output y
     (W4A4 operands with EPI_SWIGLU or y_dtype BF16 only), formed while y is
     written: amax over the stored bf16 values (NaN skipped) / 2688, 1 for an
     all-zero y -- bit for bit what quads_quantize_nvfp4 computes for y, so a
     following quads_quantize_nvfp4(y, ..., QUADS_GSCALE_GIVEN) with
     out.gscale = y_gscale skips its amax pass over y [Gist 2.2-B: fused
     kernels keep the RAC overhead small].  The GEMM's workgroups gather
     the amax in 64 workspace words (256 more workspace bytes, cleared by
     quads_moe_gemm_prepare; a QUADS_GEMM_PREPARED call relies on an earlier
     prepare of the same workspace) and a one-wave kernel enqueued after the
     GEMM folds them into y_gscale and clears them.  NULL: not computed. */
  float *y_gscale;
} quads_moe_gemm_args;

size_t quads_moe_gemm_workspace_bytes(const quads_moe_gemm_args *a);
quads_status_t quads_moe_w4a4_gemm(const quads_moe_gemm_args *a, void *stream);

/* quads_moe_gemm_prepare -- the first half of quads_moe_w4a4_gemm, split out
 * so callers can time or reuse it: builds the (expert, m-tile) list from
 * expert_offsets and, with a RAC residual, gathers the selected weight columns
 * sel_idx of every expert row into the workspace (fp16, exact e2m1 * e4m3
 * values), or for few rows per expert writes the corrected fp16 activation
 * operand there.  A following quads_moe_w4a4_gemm with flags |= QUADS_GEMM_PREPARED,
 * the same arguments and the same workspace launches only the GEMM kernel. */
quads_status_t quads_moe_gemm_prepare(const quads_moe_gemm_args *a, void *stream);

/* ---------------------------------------------------------------------------
 * quads_weight_qdq -- trainer-side fake quantization [Gist 2.1, 2.2-A]: each
 * of `batch` BF16 master matrices [rows, cols] is NVFP4-quantized with its own
 * tensor scale and dequantized back to BF16 (nearest-even of the FP32 value
 * fl32(e2m1 * fl32(dec(s) * g))), written to w_out.  If q_out is not NULL its
 * codes/scales/gscale also receive the NVFP4 tensor -- identical to
 * quads_quantize_nvfp4 on the same input (the shared path that aligns trainer
 * and rollout weights).  flags: QUADS_GSCALE_GIVEN reads the tensor scales
 * from q_out->gscale (q_out required); QUADS_SCALES_ONLY computes only the
 * tensor scales into q_out->gscale (q_out required, its codes/scales and
 * w_out_bf16 unused and may be NULL) -- the input of the fused
 * QUADS_OPERANDS_BF16_QDQ forward.
 * ------------------------------------------------------------------------- */
#define QUADS_SCALES_ONLY 4u
size_t quads_weight_qdq_workspace_bytes(int64_t batch, int64_t rows, int64_t cols);
quads_status_t quads_weight_qdq(const void *w_bf16, int64_t batch, int64_t rows, int64_t cols,
                                void *w_out_bf16, const quads_nvfp4_t *q_out, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * MoE support steps around the expert GEMM (the pages name expert routing
 * but not its mechanics; this is standard top-k softmax routing).
 *
 * quads_moe_route: logits [T, E] FP32 -> top-`top` experts per token by
 * logit (ties to the lower expert index), combine weights = softmax
 * probabilities of the chosen experts (no renormalization), and the
 * permutation that groups routed rows by (expert, token): expert_offsets
 * [E+1], row_token [T*top] (token of each routed row), inverse [T, top]
 * (routed row of each (token, slot)).  E <= 1024, 1 <= top <= min(E, 16).
 * Non-finite logits: every written id is still a valid expert in [0, E);
 * experts are taken by value descending with -0 == +0, -inf after every
 * real value, NaN after -inf, ties to the lower index (the weights of a
 * NaN row are unspecified).
 * ------------------------------------------------------------------------- */
size_t quads_moe_route_workspace_bytes(int64_t T, int32_t E);
quads_status_t quads_moe_route(const float *logits, int64_t T, int32_t E, int32_t top,
                               int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                               int32_t *row_token, int32_t *inverse, void *ws, size_t ws_bytes,
                               void *stream);

/* quads_moe_combine: out[t, :] = sum over slots j (in order) of
 * topk_w[t, j] * y[inverse[t, j], :], FP32 ([T, N]; y is [T*top, N] FP32). */
quads_status_t quads_moe_combine(const float *y, int64_t T, int32_t top, int64_t N,
                                 const int32_t *inverse, const float *topk_w, float *out,
                                 void *stream);

/* ---------------------------------------------------------------------------
 * W4A16 QAT backward of the grouped expert linear y[i] = W_qdq[e(i)] . x[t(i)]
 * [Gist 2.2-A]: the trainer's forward sees the NVFP4 fake-quantized weights
 * W_qdq (quads_weight_qdq) while the optimizer updates the bf16 masters, so
 * the gradient passes the QDQ unchanged (straight-through reading).
 *
 * quads_moe_wgrad_bf16: dw[e, n, k] = sum over the expert's routed rows i of
 * dy[i, n] * x[t(i), k], FP32 [E, N, K] (= the master gradient).  dy [R, N]
 * bf16 with rows grouped by expert_offsets [E+1] (device; offsets[E] == R);
 * x [act_rows, K] bf16 read at row_token[i] (NULL: row i).  An expert with no
 * rows gets a zero gradient.  N and K are multiples of 128, E <= 1024.  The
 * workspace (quads_moe_wgrad_workspace_bytes) holds dy and the gathered x
 * transposed, each expert's rows padded to a multiple of 64: about
 * 2 * (N + K) * (R + 63 E) bytes.  Arrays 16-byte aligned; errors as above.
 *
 * The input gradient dxr[i] = dy[i] . W_qdq[e(i)] is quads_moe_w4a4_gemm in
 * bf16-operand mode over W_qdq^T: quads_transpose_bf16(W_qdq, E, N, K, WT)
 * gives WT [E, K, N], and the GEMM with x_bf16 = dy (act_rows = R, identity
 * rows), w_bf16 = WT, N' = K, K' = N writes dxr [R, K].  Tokens read by
 * several routed rows sum theirs: quads_moe_combine with unit weights.
 *
 * quads_transpose_bf16: out[b] = in[b]^T for `batch` bf16 matrices
 * [rows, cols] -> [cols, rows]; rows and cols multiples of 8.
 * ------------------------------------------------------------------------- */
size_t quads_moe_wgrad_workspace_bytes(int64_t num_rows, int32_t num_experts, int64_t N, int64_t K);
quads_status_t quads_moe_wgrad_bf16(const void *dy_bf16, const void *x_bf16, const int32_t *row_token,
                                    const int32_t *expert_offsets, int32_t num_experts, int64_t num_rows,
                                    int64_t act_rows, int64_t N, int64_t K, float *dw, void *ws,
                                    size_t ws_bytes, void *stream);
quads_status_t quads_transpose_bf16(const void *in_bf16, int64_t batch, int64_t rows, int64_t cols,
                                    void *out_bf16, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QUADS_H */
