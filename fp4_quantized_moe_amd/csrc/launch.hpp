// Host-side launchers shared between the kernel translation units and the
// C-ABI layer (api.hip).  Arguments are validated by the caller; launchers
// only size grids and enqueue kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/quads.h"

namespace quads {

// ---- quantize.hip --------------------------------------------------------
struct QuantizeLaunch {
  const void *x;
  bool x_bf16;
  int64_t batch, rows, cols;
  uint8_t *codes;      // may be null (QDQ without export)
  uint8_t *scales;     // may be null
  float *gscale;       // [batch]; input if gscale_given else output (may be null if not given)
  bool gscale_given;
  float *scores;       // [cols] or null
  uint16_t *qdq_out;   // [batch, rows, cols] bf16 or null
  void *ws;            // partials
};
int amax_partials_per_tensor(int64_t n_elem);
size_t quantize_ws_bytes(int64_t batch, int64_t rows, int64_t cols);
hipError_t launch_quantize(const QuantizeLaunch &a, hipStream_t stream);
// The tensor scale g of each of `batch` matrices only (amax partials in ws,
// then one folding workgroup per matrix).
hipError_t launch_tensor_scales(const void *x, bool x_bf16, int64_t batch, int64_t rows, int64_t cols, float *gscale,
                                void *ws, hipStream_t stream);
// quads_quantize_nvfp4_noalloc: the amax partials (batch * P floats) in the
// library's per-device scratch array of kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
size_t quantize_partials_bytes(int64_t batch, int64_t rows, int64_t cols);
// Device address of the current device's scratch array (looked up once per
// device; no allocation).
hipError_t quantize_scratch(float **out);

// ---- rac.hip ---------------------------------------------------------------
struct RacLaunch {
  const void *x;
  bool x_bf16;
  int64_t rows, cols;
  const uint8_t *x_codes, *x_scales;
  const float *x_gscale;
  const float *scores;
  int64_t nsel, kpad;
  int32_t *sel_idx;
  uint8_t *r_codes, *r_scales;
  float *r_gscale;
  uint16_t *merged;  // [rows, cols] fp16 RAC-merged activation, or null
};
// Rows per group of the RAC row kernel (< 1: the shape does not fit in LDS).
int rac_rows_per_group(int64_t cols, int64_t kpad, bool merged = false);
hipError_t launch_rac_select(const RacLaunch &a, hipStream_t stream);
// The RAC-merged fp16 operand [rows, cols] from the NVFP4 codes of the
// activation and of its residual (the same row kernel and merge arithmetic
// as quads_rac_select_merged, reading R' instead of computing it); sel_idx
// [kpad] ascending with pad entries 0.
hipError_t launch_rac_merge_codes(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_g,
                                  const uint8_t *r_codes, const uint8_t *r_scales, const float *r_g, int64_t rows,
                                  int64_t cols, int64_t kpad, const int32_t *sel_idx, uint16_t *merged,
                                  hipStream_t stream);

// ---- gemm.hip --------------------------------------------------------------
struct GemmLaunch {
  int mode;       // 0: W4A4 (+ residual), 1: bf16 operands, 2: bf16 x QDQ(bf16 masters),
                  // 3: bf16 x NVFP4 weights decoded to their QDQ bf16 values
  int epilogue;   // 0: none, 1: swiglu
  bool y_bf16;
  int E, n_seg;
  int64_t num_rows, act_rows, N, K, kpad;
  const uint8_t *x_codes, *x_scales;
  const float *x_g;
  const uint8_t *r_codes, *r_scales;
  const float *r_g;
  const int32_t *sel_idx;
  const uint8_t *w_codes, *w_scales;
  const float *w_g;
  const uint16_t *x_bf16, *w_bf16;
  const int32_t *row_token, *expert_offsets;
  void *y;
  void *ws;
  const uint16_t *x_merged;  // caller's RAC-merged fp16 activation, or null
  int rac_form;              // QUADS_RAC_FORM_AUTO | _EXACT | _MERGED
  float *y_gscale;           // NVFP4 tensor scale of the bf16 output, formed by the GEMM, or null
};
size_t gemm_ws_bytes(const GemmLaunch &a);
// False when the W4A4 operands exceed what every kernel able to run the call
// can address (32-bit offsets of the register-staged kernels, and the
// DMA-staged kernel's shape limits K % 128, N % 128).
bool gemm_shape_supported(const GemmLaunch &a);
// The workspace words gathering the output amax behind y_gscale, or null.
uint32_t *gemm_amax_words(const GemmLaunch &a);
// After the main kernel: y_gscale from the gathered amax (no-op without it).
hipError_t launch_fold_amax(const GemmLaunch &a, hipStream_t stream);
// prepare: tile list + residual weight-column gather; main: the GEMM kernel.
hipError_t launch_gemm_prepare(const GemmLaunch &a, hipStream_t stream);
hipError_t launch_gemm_main(const GemmLaunch &a, hipStream_t stream);
// Few rows per expert (decode-shaped calls): weights read once, the RAC
// correction merged into one fp16 activation operand (gemm_small.hip).
bool gemm_use_small(const GemmLaunch &a);
size_t gemm_small_res_bytes(const GemmLaunch &a);
hipError_t launch_gemm_small_prepare(const GemmLaunch &a, uint16_t *r_dense, hipStream_t stream);
hipError_t launch_gemm_small(const GemmLaunch &a, const uint16_t *r_dense, hipStream_t stream);

// ---- route.hip -------------------------------------------------------------
size_t route_ws_bytes(int64_t T, int E);
hipError_t launch_route(const float *logits, int64_t T, int E, int top, int32_t *ids, float *w,
                        int32_t *offsets, int32_t *row_token, int32_t *inverse, void *ws,
                        hipStream_t stream);
hipError_t launch_combine(const float *y, int64_t T, int top, int64_t N, const int32_t *inverse,
                          const float *w, float *out, hipStream_t stream);

// ---- backward.hip ----------------------------------------------------------
struct WgradLaunch {
  const uint16_t *dy;  // [R, N] bf16, routed rows grouped by expert
  const uint16_t *x;   // [act_rows, K] bf16
  const int32_t *row_token, *expert_offsets;
  int E;
  int64_t R, N, K;
  float *dw;  // [E, N, K]
  void *ws;
};
int64_t wgrad_padded_cols(int64_t R, int E);
size_t wgrad_ws_bytes(int64_t R, int E, int64_t N, int64_t K);
hipError_t launch_wgrad(const WgradLaunch &a, hipStream_t stream);
hipError_t launch_transpose_bf16(const uint16_t *in, int64_t batch, int64_t rows, int64_t cols, uint16_t *out,
                                 hipStream_t stream);

}  // namespace quads
