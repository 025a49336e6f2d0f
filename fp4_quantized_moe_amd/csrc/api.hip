// C ABI of libquads (declared in include/quads.h): argument validation,
// workspace sizing, status codes and the thread-local error message.  Every
// entry point only enqueues work on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include <hip/hip_runtime.h>

#include "../../include/quads.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

quads_status_t fail(quads_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

quads_status_t ok() {
  g_err[0] = '\0';
  return QUADS_OK;
}

quads_status_t device_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(QUADS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Kernels read and write arrays with 8- and 16-byte vector accesses.
bool misaligned(std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16) return true;
  return false;
}

bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a >= 0 && b >= 0 && (a == 0 || b <= lim / a); }

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxSelectCols = 16384;

}  // namespace

extern "C" {

const char *quads_last_error(void) { return g_err; }

const char *quads_version(void) { return "quads-gfx950 0.1"; }

int64_t quads_rac_nsel(int64_t cols, int32_t k_percent) {
  if (cols < 0 || k_percent < 0 || k_percent > 100 || cols > kMaxElems) return -1;
  return cols * k_percent / 100;
}

int64_t quads_rac_kpad(int64_t nsel) {
  if (nsel < 0) return -1;
  return (nsel + 15) / 16 * 16;
}

size_t quads_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch <= 0 || rows < 0 || cols <= 0) return 0;
  return quads::quantize_ws_bytes(batch, rows, cols);
}

// Argument checks shared by quads_quantize_nvfp4 and its no-allocation
// variant; QUADS_OK with *empty set for a call with no rows (no workspace or
// scratch needed).
static quads_status_t quantize_check(const void *x, quads_dtype_t dt, const quads_nvfp4_t &out, uint32_t flags,
                                     float *scores, bool *empty) {
  *empty = false;
  if (dt != QUADS_F32 && dt != QUADS_BF16) return fail(QUADS_ERR_ARG, "quantize: bad dtype %d", dt);
  if (flags & ~(QUADS_GSCALE_GIVEN | QUADS_WANT_SCORES)) return fail(QUADS_ERR_ARG, "quantize: unknown flags");
  if (out.batch < 1 || out.rows < 0 || out.cols <= 0) return fail(QUADS_ERR_SHAPE, "quantize: bad shape");
  if (out.cols % 16) return fail(QUADS_ERR_SHAPE, "quantize: cols (%lld) must be a multiple of 16", (long long)out.cols);
  if (!mul_ok(out.rows, out.cols, kMaxElems) || !mul_ok(out.batch, out.rows * out.cols, kMaxElems))
    return fail(QUADS_ERR_SHAPE, "quantize: size overflow");
  if ((flags & QUADS_WANT_SCORES) && (out.batch != 1 || scores == nullptr))
    return fail(QUADS_ERR_ARG, "quantize: QUADS_WANT_SCORES needs batch == 1 and a scores buffer");
  if (!out.gscale) return fail(QUADS_ERR_ARG, "quantize: null gscale");
  if (out.rows == 0) {
    *empty = true;  // only the tensor scales and scores are written
    return QUADS_OK;
  }
  if (!x || !out.codes || !out.scales) return fail(QUADS_ERR_ARG, "quantize: null pointer");
  if (misaligned({x, out.codes, out.scales})) return fail(QUADS_ERR_ARG, "quantize: arrays must be 16-byte aligned");
  return QUADS_OK;
}

static quads::QuantizeLaunch quantize_launch(const void *x, quads_dtype_t dt, const quads_nvfp4_t &out,
                                             uint32_t flags, float *scores, void *ws) {
  quads::QuantizeLaunch a{};
  a.x = x;
  a.x_bf16 = dt == QUADS_BF16;
  a.batch = out.batch;
  a.rows = out.rows;
  a.cols = out.cols;
  a.codes = out.codes;
  a.scales = out.scales;
  a.gscale = out.gscale;
  a.gscale_given = (flags & QUADS_GSCALE_GIVEN) != 0;
  a.scores = (flags & QUADS_WANT_SCORES) ? scores : nullptr;
  a.qdq_out = nullptr;
  a.ws = ws;
  return a;
}

quads_status_t quads_quantize_nvfp4_noalloc(const void *x, quads_dtype_t dt, quads_nvfp4_t out, uint32_t flags,
                                            float *scores, void *stream) {
  bool empty = false;
  const quads_status_t st = quantize_check(x, dt, out, flags, scores, &empty);
  if (st != QUADS_OK) return st;
  if (empty)
    return device_status(quads::launch_quantize(quantize_launch(x, dt, out, flags, scores, nullptr),
                                                static_cast<hipStream_t>(stream)),
                         "quantize_noalloc");
  const bool given = (flags & QUADS_GSCALE_GIVEN) != 0;
  float *ws = nullptr;
  if (!given) {
    const size_t need = quads::quantize_partials_bytes(out.batch, out.rows, out.cols);
    if (need > quads::kNoAllocScratchBytes)
      return fail(QUADS_ERR_WORKSPACE,
                  "quantize_noalloc: %zu bytes of amax partials exceed the %zu-byte scratch (batch %lld; "
                  "use quads_quantize_nvfp4 with a workspace)",
                  need, quads::kNoAllocScratchBytes, (long long)out.batch);
    const hipError_t e = quads::quantize_scratch(&ws);
    if (e != hipSuccess) return device_status(e, "quantize_noalloc: scratch lookup");
  }
  return device_status(
      quads::launch_quantize(quantize_launch(x, dt, out, flags, scores, ws), static_cast<hipStream_t>(stream)),
      "quantize_noalloc");
}

quads_status_t quads_quantize_nvfp4(const void *x, quads_dtype_t dt, quads_nvfp4_t out, uint32_t flags,
                                    float *scores, void *ws, size_t ws_bytes, void *stream) {
  bool empty = false;
  const quads_status_t st = quantize_check(x, dt, out, flags, scores, &empty);
  if (st != QUADS_OK) return st;
  if (empty)
    return device_status(quads::launch_quantize(quantize_launch(x, dt, out, flags, scores, nullptr),
                                                static_cast<hipStream_t>(stream)),
                         "quantize");
  const bool given = (flags & QUADS_GSCALE_GIVEN) != 0;
  if (!given && (ws == nullptr || ws_bytes < quads::quantize_ws_bytes(out.batch, out.rows, out.cols)))
    return fail(QUADS_ERR_WORKSPACE, "quantize: workspace too small (need %zu)",
                quads::quantize_ws_bytes(out.batch, out.rows, out.cols));
  return device_status(
      quads::launch_quantize(quantize_launch(x, dt, out, flags, scores, ws), static_cast<hipStream_t>(stream)),
      "quantize");
}

size_t quads_rac_select_workspace_bytes(int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return 0;
}

static quads_status_t rac_select_impl(const char *what, const void *x, quads_dtype_t dt, const quads_nvfp4_t *xq,
                                      const float *scores, int32_t k_percent, int32_t *sel_idx, quads_nvfp4_t res,
                                      void *merged_f16, void *stream) {
  if (dt != QUADS_F32 && dt != QUADS_BF16) return fail(QUADS_ERR_ARG, "%s: bad dtype", what);
  if (!xq) return fail(QUADS_ERR_ARG, "%s: null xq", what);
  if (k_percent < 0 || k_percent > 100) return fail(QUADS_ERR_ARG, "%s: k_percent %d outside [0,100]", what, k_percent);
  if (xq->batch != 1 || xq->cols <= 0 || xq->cols % 16 || xq->rows < 0)
    return fail(QUADS_ERR_SHAPE, "%s: xq must be one [rows, cols] tensor with cols %% 16 == 0", what);
  if (xq->cols > kMaxSelectCols) return fail(QUADS_ERR_SHAPE, "%s: cols > %lld", what, (long long)kMaxSelectCols);
  const int64_t nsel = quads_rac_nsel(xq->cols, k_percent), kpad = quads_rac_kpad(nsel);
  if (res.cols != kpad || res.rows != xq->rows || res.batch != 1)
    return fail(QUADS_ERR_SHAPE, "%s: res must be [rows=%lld, kpad=%lld]", what, (long long)xq->rows, (long long)kpad);
  const bool merged = merged_f16 != nullptr;
  if (quads::rac_rows_per_group(xq->cols, kpad, merged && kpad > 0) < 1)
    return fail(QUADS_ERR_SHAPE, "%s: cols/kpad too large for the kernel's LDS staging", what);
  if (!scores || !res.gscale || (kpad > 0 && !sel_idx)) return fail(QUADS_ERR_ARG, "%s: null pointer", what);
  if (kpad > 0 && xq->rows > 0 && (!x || !xq->codes || !xq->scales || !xq->gscale || !res.codes || !res.scales))
    return fail(QUADS_ERR_ARG, "%s: null pointer", what);
  if (misaligned({x, xq->codes, xq->scales, res.codes, res.scales, scores, merged_f16}))
    return fail(QUADS_ERR_ARG, "%s: arrays must be 16-byte aligned", what);
  quads::RacLaunch a{};
  a.x = x;
  a.x_bf16 = dt == QUADS_BF16;
  a.rows = xq->rows;
  a.cols = xq->cols;
  a.x_codes = xq->codes;
  a.x_scales = xq->scales;
  a.x_gscale = xq->gscale;
  a.scores = scores;
  a.nsel = nsel;
  a.kpad = kpad;
  a.sel_idx = sel_idx;
  a.r_codes = res.codes;
  a.r_scales = res.scales;
  a.r_gscale = res.gscale;
  a.merged = static_cast<uint16_t *>(merged_f16);
  return device_status(quads::launch_rac_select(a, static_cast<hipStream_t>(stream)), what);
}

quads_status_t quads_rac_select(const void *x, quads_dtype_t dt, const quads_nvfp4_t *xq, const float *scores,
                                int32_t k_percent, int32_t *sel_idx, quads_nvfp4_t res, void *ws,
                                size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  return rac_select_impl("rac_select", x, dt, xq, scores, k_percent, sel_idx, res, nullptr, stream);
}

quads_status_t quads_rac_select_merged(const void *x, quads_dtype_t dt, const quads_nvfp4_t *xq,
                                       const float *scores, int32_t k_percent, int32_t *sel_idx, quads_nvfp4_t res,
                                       void *merged_f16, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (!merged_f16 && !(xq && xq->rows == 0))  // no rows: nothing to merge
    return fail(QUADS_ERR_ARG, "rac_select_merged: null merged_f16");
  return rac_select_impl("rac_select_merged", x, dt, xq, scores, k_percent, sel_idx, res, merged_f16, stream);
}

static quads_status_t gemm_fill(const quads_moe_gemm_args *a, quads::GemmLaunch &g) {
  if (!a) return fail(QUADS_ERR_ARG, "gemm: null args");
  if (a->struct_size != sizeof(quads_moe_gemm_args))
    return fail(QUADS_ERR_ARG, "gemm: struct_size %u != %zu", a->struct_size, sizeof(quads_moe_gemm_args));
  if (a->flags & ~QUADS_GEMM_PREPARED) return fail(QUADS_ERR_ARG, "gemm: unknown flags");
  if (a->operand_mode != QUADS_OPERANDS_W4A4 && a->operand_mode != QUADS_OPERANDS_BF16 &&
      a->operand_mode != QUADS_OPERANDS_BF16_QDQ && a->operand_mode != QUADS_OPERANDS_BF16_W4)
    return fail(QUADS_ERR_ARG, "gemm: bad operand_mode");
  if (a->epilogue != QUADS_EPI_NONE && a->epilogue != QUADS_EPI_SWIGLU) return fail(QUADS_ERR_ARG, "gemm: bad epilogue");
  if (a->y_dtype != QUADS_F32 && a->y_dtype != QUADS_BF16) return fail(QUADS_ERR_ARG, "gemm: bad y_dtype");
  if (a->num_experts < 1 || a->num_experts > 1024) return fail(QUADS_ERR_SHAPE, "gemm: num_experts outside [1,1024]");
  if (a->n_seg < 1 || a->N <= 0 || a->N % a->n_seg) return fail(QUADS_ERR_SHAPE, "gemm: bad n_seg");
  if (a->K <= 0 || a->K % 16) return fail(QUADS_ERR_SHAPE, "gemm: K must be a positive multiple of 16");
  if (a->N % 128) return fail(QUADS_ERR_SHAPE, "gemm: N must be a multiple of 128");
  if (a->epilogue == QUADS_EPI_SWIGLU && a->n_seg != 2 && a->operand_mode != QUADS_OPERANDS_BF16)
    return fail(QUADS_ERR_SHAPE, "gemm: SWIGLU needs n_seg == 2 (gate, up)");
  if (a->num_rows < 0 || a->act_rows < 0 || a->num_rows > (int64_t(1) << 31) - 1 || a->act_rows > (int64_t(1) << 31) - 1)
    return fail(QUADS_ERR_SHAPE, "gemm: row counts must fit int32");
  if (!mul_ok(a->num_rows, a->N, kMaxElems) || !mul_ok(int64_t(a->num_experts) * a->N, a->K, kMaxElems))
    return fail(QUADS_ERR_SHAPE, "gemm: size overflow");
  // No rows: y and the activation operands are not touched (they may be NULL).
  const bool rows = a->num_rows > 0;
  if (!a->expert_offsets || (rows && !a->y)) return fail(QUADS_ERR_ARG, "gemm: null expert_offsets or y");
  if (misaligned({a->y, a->ws, a->x_codes, a->x_scales, a->r_codes, a->r_scales, a->w_codes, a->w_scales, a->x_bf16,
                  a->w_bf16, a->x_merged}))
    return fail(QUADS_ERR_ARG, "gemm: arrays must be 16-byte aligned");
  if (a->row_token == nullptr && a->act_rows < a->num_rows)
    return fail(QUADS_ERR_SHAPE, "gemm: identity rows need act_rows >= num_rows");
  if (a->rac_form != QUADS_RAC_FORM_AUTO && a->rac_form != QUADS_RAC_FORM_EXACT && a->rac_form != QUADS_RAC_FORM_MERGED)
    return fail(QUADS_ERR_ARG, "gemm: bad rac_form %d", a->rac_form);
  if (a->rac_form == QUADS_RAC_FORM_EXACT && a->x_merged != nullptr)
    return fail(QUADS_ERR_ARG, "gemm: x_merged is the merged form; rac_form EXACT needs x_merged == NULL");
  if (a->y_gscale != nullptr &&
      (a->operand_mode != QUADS_OPERANDS_W4A4 || (a->epilogue != QUADS_EPI_SWIGLU && a->y_dtype != QUADS_BF16)))
    return fail(QUADS_ERR_ARG, "gemm: y_gscale needs W4A4 operands and a bf16 output (SWIGLU or y_dtype BF16)");
  g = quads::GemmLaunch{};
  g.rac_form = a->rac_form;
  g.y_gscale = a->y_gscale;
  g.mode = a->operand_mode == QUADS_OPERANDS_BF16       ? 1
           : a->operand_mode == QUADS_OPERANDS_BF16_QDQ ? 2
           : a->operand_mode == QUADS_OPERANDS_BF16_W4  ? 3
                                                        : 0;
  g.epilogue = a->epilogue;
  g.y_bf16 = a->y_dtype == QUADS_BF16;
  g.E = a->num_experts;
  g.n_seg = a->n_seg;
  g.num_rows = a->num_rows;
  g.act_rows = a->act_rows;
  g.N = a->N;
  g.K = a->K;
  g.row_token = a->row_token;
  g.expert_offsets = a->expert_offsets;
  g.y = a->y;
  g.ws = a->ws;
  if (g.mode == 0) {
    if (!a->w_codes || !a->w_scales || !a->w_gscale || (rows && (!a->x_codes || !a->x_scales || !a->x_gscale)))
      return fail(QUADS_ERR_ARG, "gemm: null W4A4 operand");
    g.x_codes = a->x_codes;
    g.x_scales = a->x_scales;
    g.x_g = a->x_gscale;
    g.w_codes = a->w_codes;
    g.w_scales = a->w_scales;
    g.w_g = a->w_gscale;
    if (a->r_codes != nullptr && a->kpad > 0) {
      if (a->kpad % 16 || a->kpad > 16384) return fail(QUADS_ERR_SHAPE, "gemm: kpad must be a multiple of 16, <= 16384");
      if (!a->r_scales || !a->r_gscale || !a->sel_idx) return fail(QUADS_ERR_ARG, "gemm: null residual operand");
      g.r_codes = a->r_codes;
      g.r_scales = a->r_scales;
      g.r_g = a->r_gscale;
      g.sel_idx = a->sel_idx;
      g.kpad = a->kpad;
      g.x_merged = static_cast<const uint16_t *>(a->x_merged);
      // The merge step stages one row of K floats plus the mask in LDS.
      if (a->rac_form == QUADS_RAC_FORM_MERGED && a->x_merged == nullptr &&
          quads::rac_rows_per_group(a->K, a->kpad, true) < 1)
        return fail(QUADS_ERR_SHAPE, "gemm: K %lld too large for the merge step (pass x_merged or rac_form EXACT)",
                    (long long)a->K);
    }
  } else if (g.mode == 3) {
    if ((rows && !a->x_bf16) || !a->w_codes || !a->w_scales || !a->w_gscale)
      return fail(QUADS_ERR_ARG, "gemm: BF16_W4 needs x_bf16 and the NVFP4 weights (w_codes, w_scales, w_gscale)");
    g.x_bf16 = static_cast<const uint16_t *>(a->x_bf16);
    g.w_codes = a->w_codes;
    g.w_scales = a->w_scales;
    g.w_g = a->w_gscale;
  } else {
    if ((rows && !a->x_bf16) || !a->w_bf16) return fail(QUADS_ERR_ARG, "gemm: null bf16 operand");
    g.x_bf16 = static_cast<const uint16_t *>(a->x_bf16);
    g.w_bf16 = static_cast<const uint16_t *>(a->w_bf16);
    if (g.mode == 2) {
      if (!a->w_gscale) return fail(QUADS_ERR_ARG, "gemm: BF16_QDQ needs the masters' tensor scales (w_gscale)");
      g.w_g = a->w_gscale;
    }
  }
  if (!quads::gemm_shape_supported(g))
    return fail(QUADS_ERR_SHAPE,
                "gemm: W4A4 activation or one expert's weights beyond 4 GiB need K %% 128 == 0 and kpad %% 64 == 0");
  return QUADS_OK;
}

size_t quads_moe_gemm_workspace_bytes(const quads_moe_gemm_args *a) {
  quads::GemmLaunch g;
  if (gemm_fill(a, g) != QUADS_OK) return 0;
  return quads::gemm_ws_bytes(g);
}

quads_status_t quads_moe_gemm_prepare(const quads_moe_gemm_args *a, void *stream) {
  quads::GemmLaunch g;
  const quads_status_t st = gemm_fill(a, g);
  if (st != QUADS_OK) return st;
  if (a->ws == nullptr || a->ws_bytes < quads::gemm_ws_bytes(g))
    return fail(QUADS_ERR_WORKSPACE, "gemm: workspace too small (need %zu)", quads::gemm_ws_bytes(g));
  return device_status(quads::launch_gemm_prepare(g, static_cast<hipStream_t>(stream)), "gemm_prepare");
}

quads_status_t quads_moe_w4a4_gemm(const quads_moe_gemm_args *a, void *stream) {
  quads::GemmLaunch g;
  const quads_status_t st = gemm_fill(a, g);
  if (st != QUADS_OK) return st;
  if (a->ws == nullptr || a->ws_bytes < quads::gemm_ws_bytes(g))
    return fail(QUADS_ERR_WORKSPACE, "gemm: workspace too small (need %zu)", quads::gemm_ws_bytes(g));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(a->flags & QUADS_GEMM_PREPARED)) {
    const hipError_t e = quads::launch_gemm_prepare(g, s);
    if (e != hipSuccess) return device_status(e, "gemm_prepare");
  }
  const hipError_t e = quads::launch_gemm_main(g, s);
  if (e != hipSuccess) return device_status(e, "gemm");
  return device_status(quads::launch_fold_amax(g, s), "gemm: output tensor scale");
}

size_t quads_weight_qdq_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
  return quads_quantize_workspace_bytes(batch, rows, cols);
}

quads_status_t quads_weight_qdq(const void *w_bf16, int64_t batch, int64_t rows, int64_t cols, void *w_out_bf16,
                                const quads_nvfp4_t *q_out, uint32_t flags, void *ws, size_t ws_bytes,
                                void *stream) {
  if (flags & ~(QUADS_GSCALE_GIVEN | QUADS_SCALES_ONLY)) return fail(QUADS_ERR_ARG, "weight_qdq: unknown flags");
  if (flags & QUADS_SCALES_ONLY) {
    if (flags & QUADS_GSCALE_GIVEN) return fail(QUADS_ERR_ARG, "weight_qdq: QUADS_SCALES_ONLY with QUADS_GSCALE_GIVEN");
    if (batch < 1 || rows < 0 || cols <= 0 || cols % 16)
      return fail(QUADS_ERR_SHAPE, "weight_qdq: bad shape (cols must be a positive multiple of 16)");
    if (!mul_ok(rows, cols, kMaxElems) || !mul_ok(batch, rows * cols, kMaxElems))
      return fail(QUADS_ERR_SHAPE, "weight_qdq: size overflow");
    if (!q_out || !q_out->gscale) return fail(QUADS_ERR_ARG, "weight_qdq: QUADS_SCALES_ONLY needs q_out->gscale");
    if (q_out->batch != batch || q_out->rows != rows || q_out->cols != cols)
      return fail(QUADS_ERR_SHAPE, "weight_qdq: q_out shape mismatch");
    if (rows > 0 && !w_bf16) return fail(QUADS_ERR_ARG, "weight_qdq: null pointer");
    if (misaligned({w_bf16})) return fail(QUADS_ERR_ARG, "weight_qdq: arrays must be 16-byte aligned");
    if (ws == nullptr || ws_bytes < quads::quantize_ws_bytes(batch, rows, cols))
      return fail(QUADS_ERR_WORKSPACE, "weight_qdq: workspace too small (need %zu)",
                  quads::quantize_ws_bytes(batch, rows, cols));
    return device_status(quads::launch_tensor_scales(w_bf16, true, batch, rows, cols, q_out->gscale, ws,
                                                     static_cast<hipStream_t>(stream)),
                         "weight_qdq");
  }
  if (batch < 1 || rows < 0 || cols <= 0 || cols % 16)
    return fail(QUADS_ERR_SHAPE, "weight_qdq: bad shape (cols must be a positive multiple of 16)");
  if (!mul_ok(rows, cols, kMaxElems) || !mul_ok(batch, rows * cols, kMaxElems))
    return fail(QUADS_ERR_SHAPE, "weight_qdq: size overflow");
  const bool given = (flags & QUADS_GSCALE_GIVEN) != 0;
  if (given && (q_out == nullptr || q_out->gscale == nullptr))
    return fail(QUADS_ERR_ARG, "weight_qdq: QUADS_GSCALE_GIVEN needs q_out->gscale");
  if (q_out && (q_out->batch != batch || q_out->rows != rows || q_out->cols != cols))
    return fail(QUADS_ERR_SHAPE, "weight_qdq: q_out shape mismatch");
  if (rows == 0) return ok();
  if (!w_bf16 || !w_out_bf16) return fail(QUADS_ERR_ARG, "weight_qdq: null pointer");
  if (misaligned({w_bf16, w_out_bf16}) || (q_out && misaligned({q_out->codes, q_out->scales})))
    return fail(QUADS_ERR_ARG, "weight_qdq: arrays must be 16-byte aligned");
  if (q_out && (!q_out->codes || !q_out->scales || !q_out->gscale)) return fail(QUADS_ERR_ARG, "weight_qdq: null q_out member");
  if (!given && (ws == nullptr || ws_bytes < quads::quantize_ws_bytes(batch, rows, cols)))
    return fail(QUADS_ERR_WORKSPACE, "weight_qdq: workspace too small (need %zu)", quads::quantize_ws_bytes(batch, rows, cols));
  quads::QuantizeLaunch a{};
  a.x = w_bf16;
  a.x_bf16 = true;
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.codes = q_out ? q_out->codes : nullptr;
  a.scales = q_out ? q_out->scales : nullptr;
  a.gscale = q_out ? q_out->gscale : nullptr;
  a.gscale_given = given;
  a.scores = nullptr;
  a.qdq_out = static_cast<uint16_t *>(w_out_bf16);
  a.ws = ws;
  return device_status(quads::launch_quantize(a, static_cast<hipStream_t>(stream)), "weight_qdq");
}

size_t quads_moe_route_workspace_bytes(int64_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return quads::route_ws_bytes(T, E);
}

quads_status_t quads_moe_route(const float *logits, int64_t T, int32_t E, int32_t top, int32_t *topk_ids,
                               float *topk_w, int32_t *expert_offsets, int32_t *row_token, int32_t *inverse,
                               void *ws, size_t ws_bytes, void *stream) {
  if (E < 1 || E > 1024) return fail(QUADS_ERR_SHAPE, "route: E outside [1,1024]");
  if (top < 1 || top > 16 || top > E) return fail(QUADS_ERR_SHAPE, "route: top outside [1, min(E,16)]");
  if (T < 0 || !mul_ok(T, top, (int64_t(1) << 31) - 1) || !mul_ok(T, E, kMaxElems))
    return fail(QUADS_ERR_SHAPE, "route: T out of range");
  if (!expert_offsets) return fail(QUADS_ERR_ARG, "route: null expert_offsets");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !row_token || !inverse)) return fail(QUADS_ERR_ARG, "route: null pointer");
  if (ws == nullptr || ws_bytes < quads::route_ws_bytes(T, E))
    return fail(QUADS_ERR_WORKSPACE, "route: workspace too small (need %zu)", quads::route_ws_bytes(T, E));
  return device_status(quads::launch_route(logits, T, E, top, topk_ids, topk_w, expert_offsets, row_token, inverse, ws,
                                           static_cast<hipStream_t>(stream)),
                       "route");
}

quads_status_t quads_moe_combine(const float *y, int64_t T, int32_t top, int64_t N, const int32_t *inverse,
                                 const float *topk_w, float *out, void *stream) {
  if (T < 0 || top < 1 || top > 16 || N <= 0 || N % 4) return fail(QUADS_ERR_SHAPE, "combine: bad shape (N %% 4 == 0)");
  if (T > 0 && (!y || !inverse || !topk_w || !out)) return fail(QUADS_ERR_ARG, "combine: null pointer");
  return device_status(quads::launch_combine(y, T, top, N, inverse, topk_w, out, static_cast<hipStream_t>(stream)),
                       "combine");
}

size_t quads_moe_wgrad_workspace_bytes(int64_t num_rows, int32_t num_experts, int64_t N, int64_t K) {
  if (num_rows < 0 || num_experts < 1 || num_experts > 1024 || N <= 0 || K <= 0) return 0;
  return quads::wgrad_ws_bytes(num_rows, num_experts, N, K);
}

quads_status_t quads_moe_wgrad_bf16(const void *dy_bf16, const void *x_bf16, const int32_t *row_token,
                                    const int32_t *expert_offsets, int32_t num_experts, int64_t num_rows,
                                    int64_t act_rows, int64_t N, int64_t K, float *dw, void *ws, size_t ws_bytes,
                                    void *stream) {
  if (num_experts < 1 || num_experts > 1024) return fail(QUADS_ERR_SHAPE, "wgrad: num_experts outside [1,1024]");
  if (N <= 0 || K <= 0 || N % 128 || K % 128) return fail(QUADS_ERR_SHAPE, "wgrad: N and K must be positive multiples of 128");
  if (num_rows < 0 || act_rows < 0 || num_rows + 63 * int64_t(num_experts) > (int64_t(1) << 31) - 64)
    return fail(QUADS_ERR_SHAPE, "wgrad: row counts out of range");
  if (!mul_ok(int64_t(num_experts) * N, K, kMaxElems) || !mul_ok(num_rows + 64 * int64_t(num_experts), N + K, kMaxElems))
    return fail(QUADS_ERR_SHAPE, "wgrad: size overflow");
  if (row_token == nullptr && act_rows < num_rows)
    return fail(QUADS_ERR_SHAPE, "wgrad: identity rows need act_rows >= num_rows");
  if (!expert_offsets || !dw || (num_rows > 0 && (!dy_bf16 || !x_bf16))) return fail(QUADS_ERR_ARG, "wgrad: null pointer");
  if (misaligned({dy_bf16, x_bf16, dw, ws})) return fail(QUADS_ERR_ARG, "wgrad: arrays must be 16-byte aligned");
  const size_t need = quads::wgrad_ws_bytes(num_rows, num_experts, N, K);
  if (ws == nullptr || ws_bytes < need) return fail(QUADS_ERR_WORKSPACE, "wgrad: workspace too small (need %zu)", need);
  quads::WgradLaunch a{};
  a.dy = static_cast<const uint16_t *>(dy_bf16);
  a.x = static_cast<const uint16_t *>(x_bf16);
  a.row_token = row_token;
  a.expert_offsets = expert_offsets;
  a.E = num_experts;
  a.R = num_rows;
  a.N = N;
  a.K = K;
  a.dw = dw;
  a.ws = ws;
  return device_status(quads::launch_wgrad(a, static_cast<hipStream_t>(stream)), "wgrad");
}

quads_status_t quads_transpose_bf16(const void *in_bf16, int64_t batch, int64_t rows, int64_t cols, void *out_bf16,
                                    void *stream) {
  if (batch < 0 || batch > 65535 || rows < 0 || cols < 0 || rows % 8 || cols % 8)
    return fail(QUADS_ERR_SHAPE, "transpose: rows and cols must be multiples of 8, batch <= 65535");
  if (!mul_ok(rows, cols, kMaxElems) || !mul_ok(batch, rows * cols, kMaxElems) || cols / 64 >= 65535)
    return fail(QUADS_ERR_SHAPE, "transpose: size overflow");
  if (batch * rows * cols == 0) return ok();
  if (!in_bf16 || !out_bf16) return fail(QUADS_ERR_ARG, "transpose: null pointer");
  if (misaligned({in_bf16, out_bf16})) return fail(QUADS_ERR_ARG, "transpose: arrays must be 16-byte aligned");
  return device_status(quads::launch_transpose_bf16(static_cast<const uint16_t *>(in_bf16), batch, rows, cols,
                                                    static_cast<uint16_t *>(out_bf16), static_cast<hipStream_t>(stream)),
                       "transpose");
}

}  // extern "C"
