// Residual Activation Compensation (RAC) on gfx950: channel mask and
// second-pass residual quantization, in one kernel.
//
// QUADS technical summary, section 2.2-B: channels whose first-pass FP4
// residual is largest get a binary mask (the top k% of channels, 50% being the
// example setting) and their residual is quantized a second time; that
// correction is added to the quantized path, so the native W4A4 GEMM still
// does most of the work.
//
// k_rac, per workgroup:
//   1. every workgroup finds the mask itself (redundant across workgroups, but
//      in parallel and without a second launch): the nsel-th largest score T
//      is built one bit at a time from the top, each step a workgroup count of
//      the FP32 score bit patterns (which order like the non-negative floats
//      they encode) at or above a candidate; channels above T plus the
//      lowest-index channels equal to T are kept and written in ascending
//      order with prefix sums over per-thread channel runs.  Workgroup 0 also
//      publishes the mask and the residual tensor scale, taken from the
//      largest score;
//   2. for a group of rows, dx = x - dq is recomputed for every channel with
//      16-element vector loads of x, codes and scales (the same FP32
//      operations as the quantizer) into LDS;
//   3. the selected channels are gathered from LDS in ascending order and
//      NVFP4-quantized in 16-element blocks with the residual tensor scale.
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Per-thread channel runs of the mask search: thread t owns channels
// [t*PER, t*PER + PER), so the selected indices come out in ascending order
// from prefix sums over threads.
template <int PER>
struct Keys {
  uint32_t k[PER];
};

// Sum of `v` over the workgroup, and the exclusive prefix of `w` over threads,
// with one barrier; `slot` holds 2 * kThreads / 64 words of LDS.
__device__ __forceinline__ void block_sum_and_scan(uint32_t v, uint32_t w, uint32_t *slot, uint32_t &v_total,
                                                   uint32_t &w_before) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int W = kThreads / 64;
  const uint32_t w_incl = wave_incl_scan(w, lane);
  uint32_t vs = v;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) vs += static_cast<uint32_t>(__shfl_xor(static_cast<int>(vs), off));
  if (lane == 63) {
    slot[wave] = vs;
    slot[W + wave] = w_incl;
  }
  __syncthreads();
  v_total = 0;
  w_before = w_incl - w;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    v_total += slot[i];
    if (i < wave) w_before += slot[W + i];
  }
}

// Number of keys >= cand over the workgroup (one barrier; `slot` alternates
// between two buffers of kThreads / 64 words so consecutive calls need no
// second barrier).
template <int PER>
__device__ __forceinline__ uint32_t block_count_ge(const Keys<PER> &ks, uint32_t cand, uint32_t *slot) {
  const int wave = threadIdx.x >> 6;
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) n += ks.k[i] >= cand;
  // Wave sum of n in [0, PER] from one ballot per bit of n (scalar popcounts,
  // no cross-lane data movement).
  constexpr int kBits = PER < 8 ? 3 : PER < 16 ? 4 : PER < 32 ? 5 : PER < 64 ? 6 : 7;
  uint32_t wsum = 0;
#pragma unroll
  for (int b = 0; b < kBits; ++b) wsum += static_cast<uint32_t>(__popcll(__ballot((n >> b) & 1u))) << b;
  if ((threadIdx.x & 63) == 0) slot[wave] = wsum;
  __syncthreads();
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) total += slot[i];
  return total;
}

// Writes the nsel selected channel indices (largest scores first by value,
// ties to the lower index) in ascending order to sel[0..nsel).  Keys are the
// FP32 score bit patterns: non-negative, so below 2^31 and ordered like the
// scores.  A threshold T is built bit by bit from the top: a bit stays set
// when at least nsel keys are >= the candidate.  Two exact shortcuts:
//  - every real key lies in [lo, hi], so the nsel-th largest does too, and it
//    shares the bits above the highest bit in which lo and hi differ; the
//    search starts below them;
//  - once exactly nsel keys are >= T, the set {keys >= T} is the selection
//    and the remaining bits cannot change it, so the search stops there.
//    The tie handling below then keeps every key equal to T.
// n_total is the number of keys >= any T <= lo: the K real keys, plus the
// zero padding keys when T is 0.
template <int PER>
__device__ void block_select(const Keys<PER> &ks, int nsel, uint32_t lo, uint32_t hi, int K, uint32_t *slots,
                             int32_t *sel) {
  const int c0 = threadIdx.x * PER;
  const uint32_t diff = lo ^ hi;
  const int top = diff ? 31 - __builtin_clz(diff) : -1;  // keys < 2^31, so top <= 30
  uint32_t T = top >= 0 ? hi & ~((2u << top) - 1u) : hi;
  uint32_t cur = T > 0 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(kThreads * PER);
  int buf = 0;
  for (int bit = top; bit >= 0 && cur != static_cast<uint32_t>(nsel); --bit) {
    const uint32_t cand = T | (1u << bit);
    const uint32_t n = block_count_ge(ks, cand, slots + buf * (kThreads / 64));
    if (n >= static_cast<uint32_t>(nsel)) {
      T = cand;
      cur = n;
    }
    buf ^= 1;
  }
  // Keys beyond K (padding) are 0 and come after every real channel: they are
  // never above T, and when T == 0 they only follow the real zeros among the
  // ties, of which there are at least need_eq, so no padding channel is kept.
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    n_gt += ks.k[i] > T;
    n_eq += ks.k[i] == T;
  }
  uint32_t gt_total, eq_before;
  block_sum_and_scan(n_gt, n_eq, slots + 2 * (kThreads / 64), gt_total, eq_before);
  const uint32_t need_eq = static_cast<uint32_t>(nsel) - gt_total;
  // Branch-free keep flags: a channel is kept if its key is above T, or equal
  // to T and among the first need_eq such channels.
  uint32_t n_keep = 0;
  {
    uint32_t e = eq_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool eq = ks.k[i] == T;
      n_keep += ks.k[i] > T || (eq && e < need_eq);
      e += eq;
    }
  }
  uint32_t unused, pos;
  block_sum_and_scan(0, n_keep, slots + 4 * (kThreads / 64), unused, pos);
  {
    __shared__ int32_t trash;
    uint32_t e = eq_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool eq = ks.k[i] == T;
      const bool kk = ks.k[i] > T || (eq && e < need_eq);
      e += eq;
      int32_t *dst = kk ? sel + pos : &trash;
      *dst = c0 + i;
      pos += kk;
    }
  }
}

// One 16-element block of x with its FP4 codes and E4M3 scale, as loaded.
template <bool BF16>
struct RawBlock {
  uint4 x[BF16 ? 2 : 4];
  uint2 codes;
  uint32_t scale;
};

template <bool BF16>
__device__ __forceinline__ void load_raw(RawBlock<BF16> &r, const void *x, const uint8_t *codes,
                                         const uint8_t *scales, int64_t blk_global) {
  constexpr int n = BF16 ? 2 : 4;
  const uint4 *p = reinterpret_cast<const uint4 *>(x) + blk_global * n;
#pragma unroll
  for (int i = 0; i < n; ++i) r.x[i] = p[i];
  r.codes = reinterpret_cast<const uint2 *>(codes)[blk_global];
  r.scale = scales[blk_global];
}

// dx = x - dq for one block (the quantizer's FP32 operations: dq = level * d
// with d = dec(scale) * g); with `xv` also the block's exact values
// X' = level * dec(scale) (units of g).
template <bool BF16>
__device__ __forceinline__ void block_dx(const RawBlock<BF16> &r, float gx, float (&dx)[16], float *xv = nullptr) {
  float v[16];
  if constexpr (BF16) {
    const uint32_t w[8] = {r.x[0].x, r.x[0].y, r.x[0].z, r.x[0].w, r.x[1].x, r.x[1].y, r.x[1].z, r.x[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = __uint_as_float(r.x[i].x);
      v[4 * i + 1] = __uint_as_float(r.x[i].y);
      v[4 * i + 2] = __uint_as_float(r.x[i].z);
      v[4 * i + 3] = __uint_as_float(r.x[i].w);
    }
  }
  const float sd = e4m3_to_f32(r.scale);
  const float d = sd * gx;
#define QUADS_DX(word, byte, i0)                                               \
  {                                                                            \
    const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, byte); \
    dx[i0] = v[i0] - e[0] * d;                                                 \
    dx[i0 + 1] = v[i0 + 1] - e[1] * d;                                         \
  }
  QUADS_DX(r.codes.x, 0, 0)
  QUADS_DX(r.codes.x, 1, 2)
  QUADS_DX(r.codes.x, 2, 4)
  QUADS_DX(r.codes.x, 3, 6)
  QUADS_DX(r.codes.y, 0, 8)
  QUADS_DX(r.codes.y, 1, 10)
  QUADS_DX(r.codes.y, 2, 12)
  QUADS_DX(r.codes.y, 3, 14)
#undef QUADS_DX
  if (xv != nullptr) {
    // X' from the code itself, so that a negative-zero code (0x8) gives -0
    // like every other dequantization here (the hardware conversion gives
    // +0 for it, which is immaterial for dx).
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = i < 8 ? r.codes.x : r.codes.y;
      xv[i] = dequant_code((w >> (4 * (i & 7))) & 0xFu, sd);
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store_dx(const RawBlock<BF16> &r, float gx, float *dst) {
  float dx[16];
  block_dx<BF16>(r, gx, dx);
  float4 *o = reinterpret_cast<float4 *>(dst);
  o[0] = make_float4(dx[0], dx[1], dx[2], dx[3]);
  o[1] = make_float4(dx[4], dx[5], dx[6], dx[7]);
  o[2] = make_float4(dx[8], dx[9], dx[10], dx[11]);
  o[3] = make_float4(dx[12], dx[13], dx[14], dx[15]);
}

// Blocks of one row group held in registers per thread: block tid + j*kThreads.
constexpr int kGroupSlots = 4;

// Phase 1 of both kernels: the mask, written ascending to sel[0..nsel) with
// sel[nsel..kpad) = -1; workgroup 0 also publishes it and the residual tensor
// scale, which is returned.  Ends with a barrier.
template <int PER>
__device__ __forceinline__ float find_mask(const uint32_t *scores, int K, int nsel, int kpad, int32_t *sel,
                                           uint32_t *slots, int32_t *sel_out, float *r_g_out) {
  const int tid = threadIdx.x;
  Keys<PER> ks;
  const int c0 = tid * PER;
  const int n_real = min(max(K - c0, 0), PER);  // multiple of 4 (K % 16 == 0)
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    // Clamped unconditional load; channels beyond K become key 0 via an
    // arithmetic mask (all ones while i < n_real).
    const uint4 v = *reinterpret_cast<const uint4 *>(scores + min(c0 + i, K - 4));
    const uint32_t m = static_cast<uint32_t>((i - n_real) >> 31);
    ks.k[i] = v.x & m;
    ks.k[i + 1] = v.y & m;
    ks.k[i + 2] = v.z & m;
    ks.k[i + 3] = v.w & m;
  }
  for (int j = nsel + tid; j < kpad; j += kThreads) sel[j] = -1;
  // Largest and smallest real key over the workgroup (slots 24..31; the
  // search uses slots 0..23).
  uint32_t mx = 0, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    mx = max(mx, ks.k[i]);
    if (i < n_real) mn = min(mn, ks.k[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off)));
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), off)));
  }
  if ((tid & 63) == 0) {
    slots[24 + (tid >> 6)] = mx;
    slots[28 + (tid >> 6)] = mn;
  }
  __syncthreads();
  uint32_t mx_total = 0, mn_total = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    mx_total = max(mx_total, slots[24 + i]);
    mn_total = min(mn_total, slots[28 + i]);
  }
  // The largest score is always selected (nsel >= 1): it sets the residual
  // tensor scale.
  if (nsel > 0) block_select(ks, nsel, mn_total, mx_total, K, slots, sel);
  __syncthreads();
  const float gr = tensor_scale_from_amax(nsel > 0 ? __uint_as_float(mx_total) : 0.0f);
  if (blockIdx.x == 0) {
    for (int j = tid; j < kpad; j += kThreads) sel_out[j] = max(sel[j], 0);
    if (tid == 0) *r_g_out = gr;
  }
  return gr;
}

// LDS: sel[kpad] int32 | dx rows [rb][K] fp32.  A row group has at most
// kGroupSlots * kThreads blocks.
//
// Schedule per workgroup: the loads of the first row group are issued before
// the mask search so that their latency overlaps it; afterwards, while group
// g is gathered and quantized, the loads of group g+1 are in flight.
template <bool BF16, int PER>
__global__ __launch_bounds__(kThreads) void k_rac(const void *x, int64_t rows, int K, const uint8_t *x_codes,
                                                  const uint8_t *x_scales, const float *x_g,
                                                  const uint32_t *scores, int nsel, int kpad, int32_t *sel_out,
                                                  float *r_g_out, uint8_t *r_codes, uint8_t *r_scales, int rb,
                                                  int rows_per_wg) {
  extern __shared__ uint4 lds_u4[];
  int32_t *sel = reinterpret_cast<int32_t *>(lds_u4);
  float *region = reinterpret_cast<float *>(lds_u4) + kpad;
  __shared__ uint32_t slots[8 * (kThreads / 64)];
  const int tid = threadIdx.x;
  const int cb = K / 16, nblk = kpad / 16;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t r_stop = min(r_begin + rows_per_wg, rows);

  // Loads of a row group starting at row r0 (nb blocks; clamped addresses,
  // slots past nb are skipped with a uniform test).
  RawBlock<BF16> raw[kGroupSlots];
  auto issue = [&](int64_t r0) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j)
      if (j * kThreads < nb) load_raw<BF16>(raw[j], x, x_codes, x_scales, r0 * cb + min(tid + j * kThreads, nb - 1));
  };
  const bool has_rows = kpad > 0 && r_begin < r_stop;
  if (has_rows) issue(r_begin);

  // 1. Mask.
  const float gr = find_mask<PER>(scores, K, nsel, kpad, sel, slots, sel_out, r_g_out);
  if (!has_rows) return;

  // 2-3. Residual rows.
  const TensorScale tsr = tensor_scale(gr);
  const float gx = *x_g;
  for (int64_t r0 = r_begin; r0 < r_stop; r0 += rb) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      const int b = tid + j * kThreads;
      if (j * kThreads < nb && b < nb) store_dx<BF16>(raw[j], gx, region + b * 16);
    }
    if (r0 + rb < r_stop) issue(r0 + rb);
    __syncthreads();
    for (int t = tid; t < nr * nblk; t += kThreads) {
      const int rr = t / nblk, jb = t - rr * nblk;
      const float *src = region + rr * K;
      float g16[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = sel[jb * 16 + i];
        g16[i] = c >= 0 ? src[c] : 0.0f;
      }
      const BlockQ q = quantize_block16(g16, tsr, nullptr);
      const int64_t row = r0 + rr;
      reinterpret_cast<uint2 *>(r_codes)[row * nblk + jb] = make_uint2(q.lo, q.hi);
      r_scales[row * nblk + jb] = static_cast<uint8_t>(q.scale);
    }
    __syncthreads();  // dx region is rewritten by the next group
  }
}

// The 16 values of a block's codes times d (d >= 0), exact in FP32, with the
// code's sign also on zeros (the negative-zero code gives -0; the hardware
// conversion alone gives +0 for it).
template <int B>
__device__ __forceinline__ void dequant_byte(uint32_t w, float d, float *v) {
  const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t sign = (w << (28 - 4 * (2 * B + u))) & 0x80000000u;  // bit 3 of nibble 2B+u
    v[u] = __uint_as_float(__float_as_uint(e[u] * d) | sign);
  }
}

__device__ __forceinline__ void dequant16(uint2 codes, float d, float (&v)[16]) {
  dequant_byte<0>(codes.x, d, v + 0);
  dequant_byte<1>(codes.x, d, v + 2);
  dequant_byte<2>(codes.x, d, v + 4);
  dequant_byte<3>(codes.x, d, v + 6);
  dequant_byte<0>(codes.y, d, v + 8);
  dequant_byte<1>(codes.y, d, v + 10);
  dequant_byte<2>(codes.y, d, v + 12);
  dequant_byte<3>(codes.y, d, v + 14);
}

// The 16 compact positions of a block's channels (32-byte aligned in LDS).
__device__ __forceinline__ void block_pos(const int16_t *p, int (&ps)[16]) {
  const uint4 a = reinterpret_cast<const uint4 *>(p)[0], b = reinterpret_cast<const uint4 *>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ps[2 * i] = static_cast<int16_t>(w[i] & 0xFFFFu);
    ps[2 * i + 1] = static_cast<int16_t>(w[i] >> 16);
  }
}

// The same mask and residual, plus the RAC-corrected activation as one fp16
// operand merged[rows, K] = fp16(X' + fl32(R' * fl32(g_r / g_x))) on the
// selected channels and X' elsewhere (units of g_x).
//
// LDS: sel[kpad] int32 | pos[K] int16 (channel -> index in sel, or -1) |
// dx [rb][kpad] fp32 of the selected channels only, in mask order.
//
// Per row group:
//   a. each thread computes dx and X' of its blocks; the selected channels'
//      dx go to their compact slots, X' stays in registers;
//   b. each residual block reads 16 consecutive slots, is quantized, and
//      leaves its correction fl32(R' * ratio) in the same slots;
//   c. each thread adds its selected channels' corrections to X', rounds once
//      to fp16 and stores its blocks (32 bytes each, consecutive blocks of a
//      row in consecutive threads).
// The LDS footprint (about 25 KB at K = 2048, k = 50%, 4 rows) and, for bf16
// input with K <= 8192, at most 128 VGPRs (4 workgroups per CU) let the 1024
// workgroups of a launch be resident at once, so the redundant mask search is
// paid once per launch, not once per round of workgroups.
template <bool BF16, int PER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BF16 && PER <= 32 ? 4 : 1))) void k_rac_merged(const void *x, int64_t rows, int K, const uint8_t *x_codes,
                                                         const uint8_t *x_scales, const float *x_g,
                                                         const uint32_t *scores, int nsel, int kpad,
                                                         int32_t *sel_out, float *r_g_out, uint8_t *r_codes,
                                                         uint8_t *r_scales, int rb, int rows_per_wg,
                                                         uint16_t *merged) {
  extern __shared__ uint4 lds_u4[];
  int32_t *sel = reinterpret_cast<int32_t *>(lds_u4);
  int16_t *pos = reinterpret_cast<int16_t *>(sel + kpad);
  float *region = reinterpret_cast<float *>(lds_u4) + kpad + (K + 7) / 8 * 4;  // pos rounded up to 16 bytes
  __shared__ uint32_t slots[8 * (kThreads / 64)];
  const int tid = threadIdx.x;
  const int cb = K / 16, nblk = kpad / 16;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t r_stop = min(r_begin + rows_per_wg, rows);

  RawBlock<BF16> raw[kGroupSlots];
  auto issue = [&](int64_t r0) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j)
      if (j * kThreads < nb) load_raw<BF16>(raw[j], x, x_codes, x_scales, r0 * cb + min(tid + j * kThreads, nb - 1));
  };
  const bool has_rows = r_begin < r_stop;
  if (has_rows) issue(r_begin);
  for (int c = tid; c < K; c += kThreads) pos[c] = -1;  // ordered before use by find_mask's barriers

  // 1. Mask, and its inverse map.
  const float gr = find_mask<PER>(scores, K, nsel, kpad, sel, slots, sel_out, r_g_out);
  if (!has_rows) return;
  for (int j = tid; j < nsel; j += kThreads) pos[sel[j]] = static_cast<int16_t>(j);
  __syncthreads();

  const TensorScale tsr = tensor_scale(gr);
  const float gx = *x_g;
  const float ratio = gr / gx;
  for (int64_t r0 = r_begin; r0 < r_stop; r0 += rb) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
    // a.
    uint2 kc[kGroupSlots];  // each slot's codes and scale, for X' in c.
    uint32_t ksc[kGroupSlots];
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      const int b = tid + j * kThreads;
      if (j * kThreads < nb && b < nb) {
        kc[j] = raw[j].codes;
        ksc[j] = raw[j].scale;
        float dx[16];
        block_dx<BF16>(raw[j], gx, dx);
        const int rr = b / cb, c0 = (b - rr * cb) * 16;
        int ps[16];
        block_pos(pos + c0, ps);
        float *dst = region + rr * kpad;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (ps[i] >= 0) dst[ps[i]] = dx[i];
      }
    }
    if (r0 + rb < r_stop) issue(r0 + rb);
    __syncthreads();
    // b.
    for (int t = tid; t < nr * nblk; t += kThreads) {
      const int rr = t / nblk, jb = t - rr * nblk;
      float *src = region + rr * kpad + jb * 16;
      float g16[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) g16[i] = jb * 16 + i < nsel ? src[i] : 0.0f;
      const BlockQ q = quantize_block16(g16, tsr, nullptr);
      const int64_t row = r0 + rr;
      reinterpret_cast<uint2 *>(r_codes)[row * nblk + jb] = make_uint2(q.lo, q.hi);
      r_scales[row * nblk + jb] = static_cast<uint8_t>(q.scale);
      float rv[16];
      dequant16(make_uint2(q.lo, q.hi), e4m3_to_f32(q.scale), rv);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (jb * 16 + i < nsel) src[i] = rv[i] * ratio;
    }
    __syncthreads();
    // c.
#pragma unroll
    for (int j = 0; j < kGroupSlots; ++j) {
      const int b = tid + j * kThreads;
      if (j * kThreads < nb && b < nb) {
        const int rr = b / cb, c0 = (b - rr * cb) * 16;
        int ps[16];
        block_pos(pos + c0, ps);
        const float *cor = region + rr * kpad;
        // X' (exact in FP32, signed zeros as coded); the selected channels
        // add their correction, one rounding.
        float xv[16];
        dequant16(kc[j], e4m3_to_f32(ksc[j]), xv);
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t pair = 0;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * i + u;
            float v = xv[e];
            if (ps[e] >= 0) v += cor[ps[e]];
            pair |= static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v))) << (16 * u);
          }
          h[i] = pair;
        }
        uint4 *q = reinterpret_cast<uint4 *>(merged + (r0 * cb + b) * 16);
        q[0] = make_uint4(h[0], h[1], h[2], h[3]);
        q[1] = make_uint4(h[4], h[5], h[6], h[7]);
      }
    }
    __syncthreads();  // the slots are rewritten by the next group
  }
}

}  // namespace

// LDS bytes of a workgroup holding rb rows.
size_t rac_lds_bytes(int64_t cols, int64_t kpad, bool merged, int64_t rb) {
  if (merged) return static_cast<size_t>(kpad * 4 + (cols + 7) / 8 * 16 + rb * kpad * 4);
  return static_cast<size_t>(kpad * 4 + rb * cols * 4);
}

int rac_rows_per_group(int64_t cols, int64_t kpad, bool merged) {
  const int64_t budget = 64 * 1024 - 64;
  int64_t rb = 4;  // ~40 KiB (plain) / ~25 KiB (merged) per workgroup at cols 2048, k 50%
  while (rb > 0 && rac_lds_bytes(cols, kpad, merged, rb) > static_cast<size_t>(budget)) --rb;
  const int64_t by_slots = static_cast<int64_t>(kGroupSlots) * kThreads / (cols / 16);
  if (rb > by_slots) rb = by_slots;  // a row group's blocks fit the per-thread load slots
  return static_cast<int>(rb);
}

namespace {
template <bool BF16, int PER>
void launch_rac_t(const RacLaunch &a, int64_t n_wg, int rb, int rows_per_wg, size_t lds, hipStream_t stream) {
  if (a.merged != nullptr)
    hipLaunchKernelGGL((k_rac_merged<BF16, PER>), dim3(n_wg), dim3(kThreads), lds, stream, a.x, a.rows,
                       static_cast<int>(a.cols), a.x_codes, a.x_scales, a.x_gscale,
                       reinterpret_cast<const uint32_t *>(a.scores), static_cast<int>(a.nsel),
                       static_cast<int>(a.kpad), a.sel_idx, a.r_gscale, a.r_codes, a.r_scales, rb, rows_per_wg,
                       a.merged);
  else
    hipLaunchKernelGGL((k_rac<BF16, PER>), dim3(n_wg), dim3(kThreads), lds, stream, a.x, a.rows,
                       static_cast<int>(a.cols), a.x_codes, a.x_scales, a.x_gscale,
                       reinterpret_cast<const uint32_t *>(a.scores), static_cast<int>(a.nsel),
                       static_cast<int>(a.kpad), a.sel_idx, a.r_gscale, a.r_codes, a.r_scales, rb, rows_per_wg);
}

template <bool BF16>
void launch_rac_per(const RacLaunch &a, int64_t n_wg, int rb, int rows_per_wg, size_t lds, hipStream_t stream) {
  const int64_t per = (a.cols + kThreads - 1) / kThreads;
  if (per <= 4)
    launch_rac_t<BF16, 4>(a, n_wg, rb, rows_per_wg, lds, stream);
  else if (per <= 8)
    launch_rac_t<BF16, 8>(a, n_wg, rb, rows_per_wg, lds, stream);
  else if (per <= 16)
    launch_rac_t<BF16, 16>(a, n_wg, rb, rows_per_wg, lds, stream);
  else if (per <= 32)
    launch_rac_t<BF16, 32>(a, n_wg, rb, rows_per_wg, lds, stream);
  else
    launch_rac_t<BF16, 64>(a, n_wg, rb, rows_per_wg, lds, stream);
}
}  // namespace

hipError_t launch_rac_select(const RacLaunch &a_in, hipStream_t stream) {
  if (a_in.cols > 64 * kThreads) return hipErrorInvalidValue;  // the API bounds cols first
  const bool merged = a_in.merged != nullptr && a_in.kpad > 0;
  RacLaunch a = a_in;
  if (!merged) a.merged = nullptr;  // nothing selected: the GEMM takes the plain path
  int rb = rac_rows_per_group(a.cols, a.kpad, merged);
  if (rb < 1) return hipErrorInvalidValue;
  int64_t n_wg = a.kpad == 0 || a.rows == 0 ? 1 : (a.rows + rb - 1) / rb;
  int rows_per_wg = rb;
  if (n_wg > 1024) {
    const int64_t iters = (n_wg + 1023) / 1024;
    rows_per_wg = static_cast<int>(rb * iters);
    n_wg = (a.rows + rows_per_wg - 1) / rows_per_wg;
  }
  const size_t lds = rac_lds_bytes(a.cols, a.kpad, merged, rb);
  if (a.x_bf16)
    launch_rac_per<true>(a, n_wg, rb, rows_per_wg, lds, stream);
  else
    launch_rac_per<false>(a, n_wg, rb, rows_per_wg, lds, stream);
  return hipGetLastError();
}

}  // namespace quads
