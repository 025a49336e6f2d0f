// Grouped W4A4 (+RAC) expert GEMM for few rows per expert (decode-shaped
// rollout batches), gfx950.
//
// With ~16 rows per expert the GEMM is bound by reading the NVFP4 weights
// once from HBM (0.5625 B per weight), and by the MFMA and decode issue of
// each weight fragment, not by the size of the contraction.  QUADS technical
// summary section 2.2-B adds the second-pass residual of the selected
// channels to the quantized activation before the GEMM
// (Y = W_q (X_q + M * dX_q)).  Here that sum is formed once per activation
// element, in units of the activation's tensor scale, by the RAC row kernel
// (from the residual codes when the caller passes the residual itself):
//
//   A[t, k] = fp16( X'[t, k] + fl32(R'[t, j] * fl32(gr / gx)) )   (k = sel_j; X' alone elsewhere)
//   Y[i, n] = gw * gx * sum_k W'[n, k] A[t(i), k]
//
// X' and R' are the exact e2m1 * e4m3 values (no tensor scale).  The
// rounding of the sum to fp16 is the only rounding besides the FP32
// accumulation: at most 2^-11 of each corrected element, which measures
// 2-3e-4 of max|Y| on the seeded workloads (the bar is 1e-3).  One MFMA per
// weight fragment instead of two, and no separate activation-code staging,
// makes this cheaper than carrying the residual as a second operand.  Plain
// W4A4 (no residual) stages and decodes the activation codes instead and is
// exact up to accumulation.
//
// k_gemm_small: a workgroup of kSW = 4 waves per (expert, 128 output
// columns); wave w owns 32 weight rows (output columns) and runs
// v_mfma_f32_32x32x16_f16 with the expert's rows (32 per pass) as the A
// operand.  A K step is 256 elements: one 128-byte line of codes per weight
// row.  Operands go from global memory straight to LDS (global_load_lds) with
// every load instruction covering whole 128-byte lines (8 lanes per line) --
// on MI355X a wave load spread over 32 rows at 32 bytes per row streams at a
// quarter of the HBM rate that whole lines reach.  Each wave stages its own
// weight rows; the activation rows (codes and scales, or the merged fp16
// operand) are staged once per workgroup, shared by its columns.  16-byte
// chunks are XOR-swizzled per row (by choosing which chunk each lane fetches)
// so that the MFMA fragment reads are bank-conflict-free.  The contraction
// order inside a step is permuted identically for both operands (lane half h
// takes elements [128h, 128h+128), 8 per MFMA).
//
// kSStages = 2 LDS stages (two workgroups per CU): step k+1 is in flight
// while step k is decoded (cvt + pk_mul, exact) and multiplied.  The loop
// handles up to four stages with partial vmcnt waits; deeper pipelines (three
// or four stages, 8-wave 256-column workgroups, one workgroup per CU) were
// measured and were not faster on the decode-shaped layer (gate_up 86-104 us
// against 83-87 us), so the weight stream is not limited by the bytes in
// flight per CU.
#include <stdlib.h>
#include <string.h>

#include "dma.hpp"
#include "fp4_mfma.hpp"
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kSK = 256;           // K per step
constexpr int kSW = 4;             // waves per workgroup
constexpr int kSBN = 32 * kSW;     // weight rows (output columns) per workgroup
constexpr int kSM = 32;            // rows per pass
constexpr int kSStages = 2;        // LDS stages

struct SmallParams {
  const int32_t *expert_offsets, *row_token;
  int E, n_tiles, n_seg;
  int64_t N, K;
  const uint8_t *x_codes, *x_scales;
  const float *x_g;
  const uint16_t *r_dense;  // [act_rows, K] fp16 merged activation (RAC), or null
  const float *r_g;
  const uint8_t *w_codes, *w_scales;
  const float *w_g;
  void *y;
  int y_bf16;
  uint32_t *amax_ws;  // zeroed words gathering the amax of bf16 y when its tensor scale is wanted, else null
};

// One LDS stage.  Rows of 128 bytes hold 8 chunks; chunk c of row r sits in
// slot c ^ ((r >> 1) & 7) (32 merged-operand chunks per row: slot c ^ (r & 15)).
// TAB: the weight block scales of the whole K come from a per-workgroup
// table loaded once (below), not with every step; only the members a form
// uses are declared, so that the merged-operand form with the table fills
// exactly half of a CU's LDS and two workgroups fit.
template <bool RES, bool TAB>
struct StageLds;
template <>
struct StageLds<true, true> {
  uint4 w[kSW * 32 * 8];            // [wave][row][slot] weight codes
  uint4 r[32 * 32];                 // [row][slot] merged fp16 activation (RAC)
};
template <>
struct StageLds<true, false> {
  uint4 w[kSW * 32 * 8];
  uint32_t ws[kSW * 32 * 4];        // [wave][row][4 words] weight block scales of the step
  uint4 r[32 * 32];
};
template <>
struct StageLds<false, true> {
  uint4 w[kSW * 32 * 8];
  uint4 x[32 * 8];                  // [row][slot] activation codes (plain W4A4)
  uint32_t xs[32 * 4];              // [row][4 words] activation block scales (plain W4A4)
};
template <>
struct StageLds<false, false> {
  uint4 w[kSW * 32 * 8];
  uint32_t ws[kSW * 32 * 4];
  uint4 x[32 * 8];
  uint32_t xs[32 * 4];
};

// The scale table.  Each wave's 32 weight rows are consecutive rows of the
// scale tensor, so their K/16 bytes each form one contiguous run of 2K
// bytes, copied with whole-line loads at the start of the workgroup.  Per K
// step the same bytes as 16-byte pieces of 32 rows on 32 lines cost more
// load time than the codes they scale (a probe of the kernel's loads alone:
// 55 us with per-step pieces, 49 us with the table, 41 us without scales).
// Row r holds CPR = K/256 chunks of 16 bytes (one per step); step c of row r
// sits at chunk c ^ ((r >> (4 - log2 CPR)) & (CPR - 1)), so the 32 rows read
// at one step spread over the LDS banks (rows 16 apart share banks: 2-way).
// K in {256, 512, 1024, 2048}.
constexpr int kSTabK = 2048;
constexpr int kSTabWords = kSW * 32 * (kSTabK / 64);

inline bool small_tab(int64_t K) { return K == 256 || K == 512 || K == 1024 || K == 2048; }

struct ScaleTab {
  int cpr_log2;  // log2(K / 256)
  __device__ __forceinline__ int chunk(int r, int c) const {
    return c ^ ((r >> (4 - cpr_log2)) & ((1 << cpr_log2) - 1));
  }
};

// Activation staging of a step is split into 8 (plain W4A4) or 16 (merged
// operand) DMA jobs, kSA per wave.  Merged operand: job j stages rows 2j and
// 2j+1 (32 chunks each); in a 16-row pass job j stages rows 2(j % 8) and
// 2(j % 8)+1, so jobs 8-15 repeat jobs 0-7.  Plain W4A4: jobs 0-3 stage the
// code lines of rows 8j..8j+7, jobs 4-5 the scale words of rows
// 16(j-4)..16(j-4)+15, jobs 6-7 repeat jobs 2-3.  Repeats write identical
// bytes to the same LDS words; they keep every wave's DMA count equal.
template <bool RES>
constexpr int kSA = (RES ? 16 : 8) / kSW;
static_assert((16 / kSW) * kSW == 16 && (8 / kSW) * kSW == 8, "activation jobs must split evenly over the waves");

// DMA instructions per wave per step: 4 weight-code lines, 2 weight-scale
// words (without the table) and the activation jobs.
template <bool RES, bool TAB>
constexpr int kSP = (TAB ? 4 : 6) + kSA<RES>;

__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// Per-lane row bookkeeping for the staging loads of one pass.
struct SmallRows {
  int64_t wrow[4];           // weight rows of this wave's 4 code loads (rows 8q + lane/8)
  int64_t wsrow[2];          // weight rows of the 2 scale loads (rows (64i + lane)/4)
  int64_t arow[16 / kSW];    // activation rows of this wave's activation jobs
};

// Pass row that lane `lane` stages in activation job j.
template <bool RES>
__device__ __forceinline__ int act_job_row(int j, int lane, bool rows16) {
  if constexpr (RES) {
    return 2 * (rows16 ? (j & 7) : j) + (lane >> 5);
  } else {
    if (j >= 4 && j < 6) return (64 * (j - 4) + lane) / 4;
    return 8 * (j & 3) + (lane >> 3);
  }
}

template <bool RES, bool TAB>
__device__ __forceinline__ void issue(StageLds<RES, TAB> &st, const SmallParams &p, const SmallRows &rw, int kt,
                                      int wave, int lane, bool rows16) {
  const int64_t K = p.K;
  const int slot = lane & 7;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int chunk = slot ^ swz8(r);
    dma(p.w_codes + rw.wrow[q] * (K / 2) + kt * 128 + chunk * 16, &st.w[(wave * 32 + 8 * q) * 8], 16);
  }
  if constexpr (!TAB) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma(p.w_scales + rw.wsrow[i] * (K / 16) + kt * 16 + (lane & 3) * 4, &st.ws[wave * 128 + 64 * i], 4);
  }
#pragma unroll
  for (int q = 0; q < kSA<RES>; ++q) {
    const int j = wave * kSA<RES> + q;  // wave-uniform
    // Repeat jobs only keep the per-wave DMA counts equal for the partial
    // waits of three or more stages; with two, every wait is vmcnt(0).
    const bool repeat = RES ? (rows16 && j >= 8) : j >= 6;
    if (kSStages == 2 && repeat) continue;
    const int r = act_job_row<RES>(j, lane, rows16);
    if constexpr (RES) {
      const int r_pair = 2 * (rows16 ? (j & 7) : j);
      const int chunk = (lane & 31) ^ (r & 15);
      dma(p.r_dense + rw.arow[q] * K + kt * 256 + chunk * 8, &st.r[r_pair * 32], 16);
    } else if (j >= 4 && j < 6) {
      dma(p.x_scales + rw.arow[q] * (K / 16) + kt * 16 + (lane & 3) * 4, &st.xs[64 * (j - 4)], 4);
    } else {
      const int chunk = slot ^ swz8(r);
      dma(p.x_codes + rw.arow[q] * (K / 2) + kt * 128 + chunk * 16, &st.x[8 * (j & 3) * 8], 16);
    }
  }
}

// This wave's part of the table: LDS chunk P of the wave (row P / CPR,
// position P % CPR) holds step chunk(row, position) of that row.
__device__ __forceinline__ void load_scale_table(uint32_t *tab, const ScaleTab &tb, const SmallParams &p,
                                                 int64_t wrow0, int wave, int lane) {
  const int cpr = 1 << tb.cpr_log2, chunks = 32 * cpr;
  uint32_t *base = tab + wave * chunks * 4;
  for (int off = 0; off < chunks; off += 64) {
    const int P = off + lane;
    const int r = P >> tb.cpr_log2, c = tb.chunk(r, P & (cpr - 1));
    if (P < chunks) dma(p.w_scales + (wrow0 + r) * (p.K / 16) + c * 16, base + off * 4, 16);
  }
}

// The 16 scale bytes of step kt for row r of this wave (4 words).
template <bool RES, bool TAB>
__device__ __forceinline__ const uint32_t *step_scales(const StageLds<RES, TAB> &st, const uint32_t *tab,
                                                       const ScaleTab &tb, int wave, int r, int kt) {
  if constexpr (TAB) return tab + ((wave * 32 + r) * (1 << tb.cpr_log2) + tb.chunk(r, kt)) * 4;
  else return &st.ws[wave * 128 + r * 4];
}

template <bool RES, bool TAB>
__device__ __forceinline__ void compute(const StageLds<RES, TAB> &st, const uint32_t *tab, const ScaleTab &tb, int kt,
                                        int wave, int lane, f32x16 &acc) {
  const int r = lane & 31, h = lane >> 5;
  const uint32_t *sw = step_scales<RES, TAB>(st, tab, tb, wave, r, kt);
  const uint32_t ws0 = sw[2 * h], ws1 = sw[2 * h + 1];
#pragma unroll
  for (int cq = 0; cq < 4; ++cq) {
    const int c = 4 * h + cq;
    const uint4 wc = st.w[(wave * 32 + r) * 8 + (c ^ swz8(r))];
    const uint32_t wv[4] = {wc.x, wc.y, wc.z, wc.w};
    uint32_t xv[4] = {0, 0, 0, 0};
    uint32_t xs0 = 0, xs1 = 0;
    if constexpr (!RES) {
      const uint4 xc = st.x[r * 8 + (c ^ swz8(r))];
      xv[0] = xc.x;
      xv[1] = xc.y;
      xv[2] = xc.z;
      xv[3] = xc.w;
      xs0 = st.xs[r * 4 + 2 * h];
      xs1 = st.xs[r * 4 + 2 * h + 1];
    }
#pragma unroll
    for (int sq = 0; sq < 4; ++sq) {
      const int s = 4 * cq + sq;                 // sub-step: elements [128h + 8s, +8)
      const int blk = s >> 1;                    // block among the lane's 8
      const uint32_t wsw = blk < 4 ? ws0 : ws1;
      const uint4 bw = decode8_f16(wv[sq], scale_h2((wsw >> (8 * (blk & 3))) & 0xFFu));
      uint4 ax;
      if constexpr (RES) {
        ax = st.r[r * 32 + ((16 * h + s) ^ (r & 15))];
      } else {
        const uint32_t xsw = blk < 4 ? xs0 : xs1;
        ax = decode8_f16(xv[sq], scale_h2((xsw >> (8 * (blk & 3))) & 0xFFu));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, ax), __builtin_bit_cast(h8, bw), acc, 0, 0,
                                                   0);
    }
  }
}

// 16-row pass (v_mfma_f32_16x16x32_f16): lane quarter q takes chunks 2q
// and 2q+1 of each 256-element step, 8 elements per MFMA; the wave's 32
// weight rows are two 16-column blocks.  Same contraction-order permutation
// for both operands (and the merged operand).
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool RES, bool TAB>
__device__ __forceinline__ void compute16(const StageLds<RES, TAB> &st, const uint32_t *tab, const ScaleTab &tb,
                                          int kt, int wave, int lane, f32x4 (&acc)[2]) {
  const int r = lane & 15, q = lane >> 4;
  uint32_t wsw[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) wsw[cb] = step_scales<RES, TAB>(st, tab, tb, wave, 16 * cb + r, kt)[q];
#pragma unroll
  for (int cq = 0; cq < 2; ++cq) {
    const int c = 2 * q + cq;
    uint4 wc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int wr = 16 * cb + r;
      wc[cb] = st.w[(wave * 32 + wr) * 8 + (c ^ swz8(wr))];
    }
    uint32_t xv[4] = {0, 0, 0, 0};
    uint32_t xsw = 0;
    if constexpr (!RES) {
      const uint4 xc = st.x[r * 8 + (c ^ swz8(r))];
      xv[0] = xc.x;
      xv[1] = xc.y;
      xv[2] = xc.z;
      xv[3] = xc.w;
      xsw = st.xs[r * 4 + q];  // blocks 4q..4q+3 of the step
    }
#pragma unroll
    for (int sq = 0; sq < 4; ++sq) {
      const int blk = 2 * cq + (sq >> 1);  // block among the lane's 4
      uint4 ax;
      if constexpr (RES)
        ax = st.r[r * 32 + ((8 * q + 4 * cq + sq) ^ r)];
      else
        ax = decode8_f16(xv[sq], scale_h2((xsw >> (8 * blk)) & 0xFFu));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint32_t wv[4] = {wc[cb].x, wc[cb].y, wc[cb].z, wc[cb].w};
        const uint4 bw = decode8_f16(wv[sq], scale_h2((wsw[cb] >> (8 * blk)) & 0xFFu));
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, ax), __builtin_bit_cast(h8, bw),
                                                         acc[cb], 0, 0, 0);
      }
    }
  }
}

// Stores one output; returns |stored value| for bf16 output (0 for FP32).
__device__ __forceinline__ float store_out(const SmallParams &p, int64_t row, int64_t col, int64_t ld, float v) {
  if (p.y_bf16) {
    const uint32_t hb = f32_to_bf16_bits(v);
    static_cast<uint16_t *>(p.y)[row * ld + col] = static_cast<uint16_t>(hb);
    return fabsf(bf16_bits_to_f32(hb));
  }
  static_cast<float *>(p.y)[row * ld + col] = v;  // few rows: y stays in the caches for the combine
  return 0.0f;
}

// h = silu(g) * u stored as bf16; returns |stored value|.
__device__ __forceinline__ float store_swiglu(const SmallParams &p, int64_t idx, float g, float u) {
  const uint32_t hb = f32_to_bf16_bits(silu(g) * u);
  static_cast<uint16_t *>(p.y)[idx] = static_cast<uint16_t>(hb);
  return fabsf(bf16_bits_to_f32(hb));
}

// The K loop of one pass over the kSStages LDS stages: steps kt+1 ..
// kt+kSStages-2 are in flight while step kt is multiplied by `comp(stage)`.
// Step s lives in stage s % kSStages; step kt+kSStages-1 is issued into the
// stage step kt-1 used, after the barrier that follows every wave's last read
// of it.
template <bool RES, bool TAB, class Comp>
__device__ __forceinline__ void stream_k(StageLds<RES, TAB> (&st)[kSStages], const SmallParams &p,
                                         const SmallRows &rw, int nk, int wave, int lane, bool rows16, Comp comp) {
  constexpr int P = kSP<RES, TAB>;
  static_assert(kSStages >= 2 && kSStages <= 4, "stages");
#pragma unroll
  for (int s = 0; s < kSStages - 1; ++s)
    if (s < nk) issue<RES, TAB>(st[s], p, rw, s, wave, lane, rows16);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's part of step kt has landed once at most its loads of the
    // steps issued after kt are outstanding ...
    const int ahead = min(kSStages - 2, nk - 1 - kt);
    if (ahead >= 2) wait_vm<2 * P>();
    else if (ahead == 1) wait_vm<P>();
    else wait_vm<0>();
    barrier_no_fence();  // ... and every wave's part; step kt-1 is no longer read
    const int nxt = kt + kSStages - 1;
    if (nxt < nk) {
      const int b = cur + kSStages - 1 >= kSStages ? cur - 1 : cur + kSStages - 1;
      issue<RES, TAB>(st[b], p, rw, nxt, wave, lane, rows16);
    }
    comp(st[cur], kt);
    cur = cur + 1 == kSStages ? 0 : cur + 1;
  }
}

// EPI 0: Y fp32/bf16 [rows, N].  EPI 1 (SwiGLU): the first half of the waves
// own gate columns and the second half the matching up columns;
// h = silu(gate) * up -> bf16 [rows, N/2].
template <int EPI, bool RES, bool TAB>
__global__ __launch_bounds__(kSW * 64, kSStages == 2 ? 2 : 1) void k_gemm_small(SmallParams p) {
  __shared__ StageLds<RES, TAB> st[kSStages];
  __shared__ uint32_t tab[TAB ? kSTabWords : 1];
  const int e = blockIdx.x / p.n_tiles, nt = blockIdx.x % p.n_tiles;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = p.expert_offsets[e], mend = p.expert_offsets[e + 1];
  if (m0 >= mend) return;
  float hmax = 0.0f;  // largest |stored bf16 value| (NaN skipped), for the output's tensor scale

  // First weight row (output column) of this wave.
  int64_t col0, wcol0;
  if constexpr (EPI == 0) {
    col0 = static_cast<int64_t>(nt) * kSBN + 32 * wave;
    wcol0 = col0;
  } else {
    col0 = static_cast<int64_t>(nt) * (kSBN / 2) + 32 * (wave % (kSW / 2));
    wcol0 = (wave / (kSW / 2)) * (p.N / 2) + col0;
  }
  const int64_t wrow0 = static_cast<int64_t>(e) * p.N + wcol0;
  const float gw = p.w_g[e * p.n_seg + static_cast<int>(wcol0) / static_cast<int>(p.N / p.n_seg)];
  const float gx = *p.x_g;
  const int nk = static_cast<int>(p.K / kSK);
  const ScaleTab tb{nk == 8 ? 3 : nk == 4 ? 2 : nk == 2 ? 1 : 0};
  if constexpr (TAB) load_scale_table(tab, tb, p, wrow0, wave, lane);  // waited for with step 0's loads

  auto act_row = [&](int pm, int r) -> int64_t {
    const int i = min(pm + r, mend - 1);  // rows past the expert re-read a valid row, never stored
    return p.row_token ? static_cast<int64_t>(p.row_token[i]) : static_cast<int64_t>(i);
  };

  for (int pm = m0; pm < mend; pm += kSM) {
    const bool rows16 = mend - pm <= 16;  // last pass of at most 16 rows: 16-row MFMAs, half the work
    SmallRows rw;
#pragma unroll
    for (int q = 0; q < 4; ++q) rw.wrow[q] = wrow0 + 8 * q + (lane >> 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) rw.wsrow[i] = wrow0 + (64 * i + lane) / 4;
#pragma unroll
    for (int q = 0; q < kSA<RES>; ++q) rw.arow[q] = act_row(pm, act_job_row<RES>(wave * kSA<RES> + q, lane, rows16));

    __syncthreads();  // the previous pass (or its epilogue) no longer reads the stages
    if (rows16) {
      f32x4 ax[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) ax[cb][v] = 0.0f;
      stream_k<RES, TAB>(st, p, rw, nk, wave, lane, true,
                         [&](const StageLds<RES, TAB> &s, int kt) __attribute__((always_inline)) {
                           compute16<RES, TAB>(s, tab, tb, kt, wave, lane, ax);
                         });
      // Element v of accumulator cb is row 4*(lane/16) + v of the pass,
      // column 16*cb + lane%16 of the wave's 32.
      const int q = lane >> 4;
      float v16[2][4];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) v16[cb][v] = ax[cb][v] * (gw * gx);  // the merged operand is in units of gx too
      if constexpr (EPI == 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = pm + 4 * q + v;
            if (row < mend) hmax = fmaxf(hmax, store_out(p, row, col0 + 16 * cb + (lane & 15), p.N, v16[cb][v]));
          }
      } else {
        float *up = reinterpret_cast<float *>(st[0].w);  // free after the K loop
        __syncthreads();
        if (wave >= kSW / 2) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int v = 0; v < 4; ++v) up[(((wave - kSW / 2) * 2 + cb) * 4 + v) * 64 + lane] = v16[cb][v];
        }
        __syncthreads();
        if (wave < kSW / 2) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int row = pm + 4 * q + v;
              const float u = up[((wave * 2 + cb) * 4 + v) * 64 + lane];
              const float g = v16[cb][v];
              if (row < mend)
                hmax = fmaxf(hmax, store_swiglu(p, static_cast<int64_t>(row) * (p.N / 2) + col0 + 16 * cb + (lane & 15),
                                                g, u));
            }
        }
      }
      continue;
    }

    f32x16 acc_x;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_x[r] = 0.0f;
    stream_k<RES, TAB>(st, p, rw, nk, wave, lane, false,
                       [&](const StageLds<RES, TAB> &s, int kt) __attribute__((always_inline)) {
                         compute<RES, TAB>(s, tab, tb, kt, wave, lane, acc_x);
                       });

    // Element r of the accumulator is row 8*(r/4) + 4*h + r%4 of the pass,
    // column lane%32 of the wave's 32.
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = acc_x[r] * (gw * gx);  // merged operand: units of gx too
    const int64_t col = col0 + (lane & 31);
    if constexpr (EPI == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = pm + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < mend) hmax = fmaxf(hmax, store_out(p, row, col, p.N, v[r]));
      }
    } else {
      float *up = reinterpret_cast<float *>(st[0].w);  // 16 KB of stage 0, free after the K loop
      __syncthreads();
      if (wave >= kSW / 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) up[((wave - kSW / 2) * 16 + r) * 64 + lane] = v[r];
      }
      __syncthreads();
      if (wave < kSW / 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = pm + 8 * (r >> 2) + 4 * h + (r & 3);
          const float u = up[(wave * 16 + r) * 64 + lane];
          const float g = v[r];
          if (row < mend) hmax = fmaxf(hmax, store_swiglu(p, static_cast<int64_t>(row) * (p.N / 2) + col, g, u));
        }
      }
    }
  }
  if (p.amax_ws != nullptr) {
    if constexpr (TAB) {
      __syncthreads();  // every wave is done with the table, which takes the per-wave partials
      amax_gather(p.amax_ws, hmax, tab);
    } else {
      amax_gather(p.amax_ws, hmax);
    }
  }
}

}  // namespace

bool gemm_use_small(const GemmLaunch &a) {
  // K in whole 256-element steps, N in whole 256-column workgroup tiles
  if (a.mode != 0 || a.K % kSK != 0 || a.K > 16384 || a.N % kSBN != 0) return false;
  // This kernel adds the RAC correction to the activation operand only (one
  // fp16 operand); the exact form runs on the many-rows kernels.
  if (a.rac_form == QUADS_RAC_FORM_EXACT && a.r_codes != nullptr && a.kpad > 0) return false;
  return a.num_rows <= static_cast<int64_t>(kSM) * a.E;  // about one pass of rows per expert
}

size_t gemm_small_res_bytes(const GemmLaunch &a) {
  return static_cast<size_t>(a.act_rows) * static_cast<size_t>(a.K) * sizeof(uint16_t);
}

hipError_t launch_gemm_small_prepare(const GemmLaunch &a, uint16_t *r_dense, hipStream_t stream) {
  if (a.r_codes == nullptr || a.kpad == 0 || a.act_rows == 0) return hipSuccess;
  return launch_rac_merge_codes(a.x_codes, a.x_scales, a.x_g, a.r_codes, a.r_scales, a.r_g, a.act_rows, a.K, a.kpad,
                                a.sel_idx, r_dense, stream);
}

hipError_t launch_gemm_small(const GemmLaunch &a, const uint16_t *r_dense, hipStream_t stream) {
  SmallParams p{};
  p.expert_offsets = a.expert_offsets;
  p.row_token = a.row_token;
  p.E = a.E;
  p.n_seg = a.n_seg;
  p.N = a.N;
  p.K = a.K;
  p.n_tiles = static_cast<int>(a.N / kSBN);
  p.x_codes = a.x_codes;
  p.x_scales = a.x_scales;
  p.x_g = a.x_g;
  p.r_dense = r_dense;
  p.r_g = a.r_g;
  p.w_codes = a.w_codes;
  p.w_scales = a.w_scales;
  p.w_g = a.w_g;
  p.y = a.y;
  p.y_bf16 = a.y_bf16 ? 1 : 0;
  p.amax_ws = gemm_amax_words(a);
  const bool res = r_dense != nullptr;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.E) * p.n_tiles)), block(kSW * 64);
  const bool tab = small_tab(a.K);
  if (a.epilogue == 0) {
    if (res && tab) hipLaunchKernelGGL((k_gemm_small<0, true, true>), grid, block, 0, stream, p);
    else if (res) hipLaunchKernelGGL((k_gemm_small<0, true, false>), grid, block, 0, stream, p);
    else if (tab) hipLaunchKernelGGL((k_gemm_small<0, false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_gemm_small<0, false, false>), grid, block, 0, stream, p);
  } else {
    if (res && tab) hipLaunchKernelGGL((k_gemm_small<1, true, true>), grid, block, 0, stream, p);
    else if (res) hipLaunchKernelGGL((k_gemm_small<1, true, false>), grid, block, 0, stream, p);
    else if (tab) hipLaunchKernelGGL((k_gemm_small<1, false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_gemm_small<1, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace quads
