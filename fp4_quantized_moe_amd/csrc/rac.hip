// Residual Activation Compensation (RAC) on gfx950: channel mask,
// second-pass residual quantization and the merged fp16 operand.
//
// QUADS technical summary, section 2.2-B: channels whose first-pass FP4
// residual is largest get a binary mask (the top k% of channels, 50% being the
// example setting) and their residual is quantized a second time; that
// correction is added to the quantized path, so the native W4A4 GEMM still
// does most of the work.
//
// Two launches per call.
//
// k_rac_mask, one workgroup: the nsel-th largest score T by radix select on
// the FP32 score bit patterns (which order like the non-negative floats they
// encode), 8 bits per round with one LDS histogram and one barrier per
// round; channels above T plus the lowest-index channels equal to T are kept
// and written in ascending order with prefix sums over per-thread channel
// runs.  It also writes the residual tensor scale, taken from the largest
// score.
//
// k_rac_rows, per group of rows:
//   a. dx = x - dq for every channel (the quantizer's FP32 operations), from
//      16-element vector loads of x, codes and scales, into a dense LDS row;
//   b. each residual block (16 consecutive mask entries) gathers its
//      channels' dx, is NVFP4-quantized with the residual tensor scale and
//      written out; for the merged operand its corrections fl32(R' * ratio)
//      go back to the same LDS slots;
//   c. (merged operand) each thread turns its blocks into fp16 from X' (its
//      codes), the mask bitmap and the corrections.
// The loads of the next group are in flight while a group is processed.  The
// same kernel, reading the residual codes in b instead of computing them,
// builds the merged operand for a GEMM that is handed the residual, so one
// code path defines that operand.
#include <algorithm>

#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kThreads = 256;

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
  const uint32_t w_incl = wave_scan<false>(w);
  const uint32_t vs = last_lane(wave_scan<false>(v));
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

// The nsel-th largest key T (nsel >= 1) by radix select, 8 bits per round
// from the top: each round counts the keys whose bits above the current digit
// equal the prefix found so far into a 256-bin LDS histogram (keys < 2^31, so
// round 0 sees 7 bits), and the digit is the bin where the count of keys at
// or above it first reaches the number still needed.  Every wave scans the
// whole histogram itself, so a round costs one barrier; each round has its
// own histogram (zeroed before the first barrier), so no round waits for the
// previous one's readers.  When the crossing bin holds exactly the keys still
// needed, every key with that prefix is kept and T is the bin's lower bound.
template <int PER>
__device__ __forceinline__ uint32_t radix_threshold(const Keys<PER> &ks, int n_real, uint32_t nsel,
                                                    uint32_t (*hist)[256]) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, need = nsel;
  for (int r = 0; r < 4; ++r) {
    const int shift = 24 - 8 * r;
    uint32_t *h = hist[r];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t key = ks.k[i];
      if (i < n_real && (static_cast<uint64_t>(key) >> (shift + 8)) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // lane l holds bins 4l..4l+3: suffix sums within the lane, then over lanes
    const uint4 b = reinterpret_cast<const uint4 *>(h)[lane];
    const uint32_t s3 = b.w, s2 = b.z + s3, s1 = b.y + s2, s0 = b.x + s1;
    const uint32_t incl_lanes = wave_scan<false>(s0);  // lanes 0..l
    const uint32_t above = last_lane(incl_lanes) - incl_lanes;  // keys in the bins above this lane's
    const uint32_t incl[4] = {above + s0, above + s1, above + s2, above + s3};
    const uint32_t cnt[4] = {b.x, b.y, b.z, b.w};
    int dsel = -1;
    uint32_t excl = 0, c = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)  // exactly one bin over the wave qualifies
      if (incl[q] >= need && incl[q] - cnt[q] < need) {
        dsel = 4 * lane + q;
        excl = incl[q] - cnt[q];
        c = cnt[q];
      }
    const int src = (__ffsll(static_cast<unsigned long long>(__ballot(dsel >= 0))) - 1) & 63;
    const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(dsel, src)) & 255u;
    need -= static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(excl), src));
    c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(c), src));
    prefix = (prefix << 8) | d;
    if (c == need) return prefix << shift;
  }
  return prefix;
}

// Emits the nsel selected channel indices (largest scores first by value,
// ties to the lower index) as emit(position, channel), positions 0..nsel-1 in
// ascending channel order.  Keys are
// the FP32 score bit patterns: non-negative, so below 2^31 and ordered like
// the scores.  Keys beyond K (padding) are 0 and come after every real
// channel: they are never above T, and when T == 0 they only follow the real
// zeros among the ties, of which there are at least need_eq, so no padding
// channel is kept.
template <int PER, class Emit>
__device__ __forceinline__ void block_select(const Keys<PER> &ks, int n_real, int nsel, uint32_t (*hist)[256],
                                             uint32_t *slots, Emit emit) {
  const int c0 = threadIdx.x * PER;
  const uint32_t T = radix_threshold<PER>(ks, n_real, static_cast<uint32_t>(nsel), hist);
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    n_gt += ks.k[i] > T;
    n_eq += ks.k[i] == T;
  }
  uint32_t gt_total, eq_before;
  block_sum_and_scan(n_gt, n_eq, slots, gt_total, eq_before);
  const uint32_t need_eq = static_cast<uint32_t>(nsel) - gt_total;
  // A channel is kept if its key is above T, or equal to T and among the
  // first need_eq such channels.
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
  block_sum_and_scan(0, n_keep, slots + 2 * (kThreads / 64), unused, pos);
  uint32_t e = eq_before;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool eq = ks.k[i] == T;
    const bool kk = ks.k[i] > T || (eq && e < need_eq);
    e += eq;
    if (kk && pos < static_cast<uint32_t>(nsel)) emit(pos, c0 + i);
    pos += kk;
  }
}

// The whole mask computed by one workgroup of kThreads threads: the channel
// scores are loaded (PER per thread), the selection is emitted through
// `emit`, and the largest key (the largest score) is returned.  `hist` and
// `slots` are the workgroup's LDS scratch.  Ends after a barrier when
// nsel > 0 (the selection's scans).
template <int PER, class Emit>
__device__ __forceinline__ uint32_t workgroup_mask(const uint32_t *scores, int K, int nsel, uint32_t (*hist)[256],
                                                   uint32_t *slots, Emit emit) {
  static_assert(kThreads == 256, "one histogram bin per thread when zeroing");
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
#pragma unroll
  for (int r = 0; r < 4; ++r) hist[r][tid] = 0;
  // Largest key over the workgroup (slots 16..19; the selection's scans use
  // slots 0..15).
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mx = max(mx, ks.k[i]);
  mx = last_lane(wave_scan<true>(mx));
  if ((tid & 63) == 0) slots[4 * (kThreads / 64) + (tid >> 6)] = mx;
  __syncthreads();
  uint32_t mx_total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) mx_total = max(mx_total, slots[4 * (kThreads / 64) + i]);
  if (nsel > 0) block_select<PER>(ks, n_real, nsel, hist, slots, emit);
  return mx_total;
}

// The mask, written ascending to sel_out[0..nsel) with pad entries
// sel_out[nsel..kpad) = 0, and the residual tensor scale (from the largest
// score, which is always selected when nsel >= 1).  One workgroup.
template <int PER>
__global__ __launch_bounds__(kThreads) void k_rac_mask(const uint32_t *scores, int K, int nsel, int kpad,
                                                       int32_t *sel_out, float *r_g_out) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t slots[6 * (kThreads / 64)];
  for (int j = nsel + threadIdx.x; j < kpad; j += kThreads) sel_out[j] = 0;
  const uint32_t mx = workgroup_mask<PER>(scores, K, nsel, hist, slots,
                                          [&](uint32_t pos, int c) { sel_out[pos] = c; });
  if (threadIdx.x == 0) *r_g_out = tensor_scale_from_amax(nsel > 0 ? __uint_as_float(mx) : 0.0f);
}

// One 16-element block of x with its FP4 codes and E4M3 scale, as loaded
// (x only when the kernel computes dx).
template <bool BF16>
struct RawBlock {
  uint4 x[BF16 ? 2 : 4];
  uint2 codes;
  uint32_t scale;
};

template <bool BF16, bool WITH_X>
__device__ __forceinline__ void load_raw(RawBlock<BF16> &r, const void *x, const uint8_t *codes,
                                         const uint8_t *scales, int64_t blk_global) {
  if constexpr (WITH_X) {
    constexpr int n = BF16 ? 2 : 4;
    const uint4 *p = reinterpret_cast<const uint4 *>(x) + blk_global * n;
#pragma unroll
    for (int i = 0; i < n; ++i) r.x[i] = p[i];
  }
  r.codes = reinterpret_cast<const uint2 *>(codes)[blk_global];
  r.scale = scales[blk_global];
}

// Dense LDS rows hold each 16-element block as four 16-byte chunks, chunk q
// of the row's block cb at position q ^ ((cb >> 2) & 3): consecutive lanes,
// which take consecutive blocks, then spread a chunk access over all banks.
__device__ __forceinline__ int chunk_pos(int cblk, int q) { return q ^ ((cblk >> 2) & 3); }

// Float offset of channel c inside its dense LDS row (0 only for c == 0).
__device__ __forceinline__ int chan_offset(int c) {
  return (c & ~15) + chunk_pos(c >> 4, (c >> 2) & 3) * 4 + (c & 3);
}

// dx = x - dq for one block (the quantizer's FP32 operations: dq = level * d
// with d = dec(scale) * g), stored as block cblk of the row at `row`.
template <bool BF16>
__device__ __forceinline__ void store_dx(const RawBlock<BF16> &r, float gx, float *row, int cblk) {
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
  float dq[16];
  const float d = e4m3_to_f32(r.scale) * gx;
  dequant8(r.codes.x, d, dq);
  dequant8(r.codes.y, d, dq + 8);
  float4 *o = reinterpret_cast<float4 *>(row + cblk * 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[chunk_pos(cblk, q)] = make_float4(v[4 * q] - dq[4 * q], v[4 * q + 1] - dq[4 * q + 1], v[4 * q + 2] - dq[4 * q + 2],
                       v[4 * q + 3] - dq[4 * q + 3]);
}

// Blocks of one row group held in registers per thread: block tid + j*kThreads
// for j < SLOTS (2 when a row has at most 512 blocks, else 4).
constexpr int kMaxSlots = 4;

// What the row kernel computes.
enum RowsMode {
  kResidual = 0,   // residual codes only (quads_rac_select)
  kMerged = 1,     // residual codes and the merged operand (quads_rac_select_merged)
  kFromCodes = 2,  // the merged operand from given residual codes (GEMM merge step)
};

struct RowsArgs {
  const void *x;  // activation (not read in kFromCodes)
  int64_t rows;
  int K, kpad;
  const uint8_t *x_codes, *x_scales;
  const float *x_g;
  const int32_t *sel;  // [kpad] ascending, pad entries 0 (mask from a previous launch)
  const float *r_g;
  // In-workgroup mask (MASK_PER > 0): the scores and nsel; workgroup 0
  // publishes the mask to sel_out and the residual tensor scale to r_g_out.
  const uint32_t *scores;
  int nsel;
  int32_t *sel_out;
  float *r_g_out;
  uint8_t *r_codes, *r_scales;  // written, or read in kFromCodes
  uint16_t *merged;              // [rows, K] fp16, or null in kResidual
  int rb, rows_per_wg;
};

// Mask bitmap words (one bit per channel), rounded up to 16 bytes.
__host__ __device__ constexpr int bitmap_words(int64_t K) { return static_cast<int>((K + 127) / 128 * 4); }

// LDS: sel[kpad] uint16 (each mask entry's offset in a dense row) | bitmap
// (merged operand only) | dense rows [rb][K] fp32 (dx, and after b the
// corrections on the selected channels).  A row group has at most SLOTS *
// kThreads blocks.  The real mask entries are the first n_real: entry 0, and
// every later entry up to the last nonzero one (nsel >= 1 whenever kpad > 0,
// the real entries ascend and the pads are 0).  An entry >= K (possible only
// in a caller's mask handed to the GEMM) is read as channel 0, so no LDS
// access leaves the rows.
//
// MASK_PER > 0 (calls of at most one workgroup per CU): every workgroup
// computes the mask itself from the scores (workgroup_mask, PER = MASK_PER
// channels per thread), with its row loads already in flight, instead of
// waiting for a mask launch; workgroup 0 publishes it.
template <bool BF16, int MODE, int SLOTS, int MASK_PER>
__global__ __launch_bounds__(kThreads) void k_rac_rows(RowsArgs p) {
  constexpr bool kX = MODE != kFromCodes;    // reads x and computes the residual
  constexpr bool kOut = MODE != kResidual;   // writes the merged operand
  extern __shared__ uint4 lds_u4[];
  const int K = p.K, kpad = p.kpad, rb = p.rb;
  uint16_t *sel = reinterpret_cast<uint16_t *>(lds_u4);
  uint32_t *bits = reinterpret_cast<uint32_t *>(sel + kpad);  // kpad % 16 == 0: 32-byte aligned
  float *region = reinterpret_cast<float *>(bits + (kOut ? bitmap_words(K) : 0));
  const int tid = threadIdx.x;
  const int cb = K / 16, nblk = kpad / 16;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_wg;
  const int64_t r_stop = min(r_begin + p.rows_per_wg, p.rows);  // > r_begin: the grid covers rows exactly

  // Loads of a row group starting at row r0 (nb blocks; clamped addresses,
  // slots past nb are skipped with a uniform test).
  RawBlock<BF16> raw[SLOTS];
  auto issue = [&](int64_t r0) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j)
      if (j * kThreads < nb)
        load_raw<BF16, kX>(raw[j], p.x, p.x_codes, p.x_scales, r0 * cb + min(tid + j * kThreads, nb - 1));
  };
  issue(r_begin);

  int n_real;
  float gr;
  if constexpr (MASK_PER > 0) {
    __shared__ uint32_t hist[4][256];
    __shared__ uint32_t mslots[6 * (kThreads / 64)];
    const bool pub = blockIdx.x == 0;
    for (int j = p.nsel + tid; j < kpad; j += kThreads) {
      sel[j] = 0;
      if (pub) p.sel_out[j] = 0;
    }
    if constexpr (kOut)
      for (int w = tid; w < bitmap_words(K); w += kThreads) bits[w] = 0;
    // (the bitmap is cleared before workgroup_mask's first barrier, which
    // precedes every emit)
    const uint32_t mx = workgroup_mask<MASK_PER>(p.scores, K, p.nsel, hist, mslots, [&](uint32_t pos, int c) {
      sel[pos] = static_cast<uint16_t>(chan_offset(c));
      if constexpr (kOut) atomicOr(&bits[c >> 5], 1u << (c & 31));
      if (pub) p.sel_out[pos] = c;
    });
    gr = tensor_scale_from_amax(__uint_as_float(mx));  // nsel >= 1 here
    if (pub && tid == 0) *p.r_g_out = gr;
    n_real = p.nsel;
    __syncthreads();
  } else {
    __shared__ int s_nreal;
    if (tid == 0) s_nreal = 1;
    if constexpr (kOut)
      for (int w = tid; w < bitmap_words(K); w += kThreads) bits[w] = 0;
    __syncthreads();
    uint32_t last = 0;  // 1 + this thread's last nonzero entry
    for (int j = tid; j < kpad; j += kThreads) {
      int c = p.sel[j];
      c = c >= 0 && c < K ? c : 0;
      sel[j] = static_cast<uint16_t>(chan_offset(c));  // < K <= 16384
      if (c != 0) last = j + 1;
      if constexpr (kOut)
        if (j == 0 || c != 0) atomicOr(&bits[c >> 5], 1u << (c & 31));
    }
    last = last_lane(wave_scan<true>(last));
    if ((tid & 63) == 0 && last > 1) atomicMax(&s_nreal, static_cast<int>(last));
    __syncthreads();
    n_real = s_nreal;
    gr = *p.r_g;
  }
  // (sel is read in b after at least one barrier; the bitmap in c after the
  // barrier that ends b.)
  const float gx = *p.x_g;
  const TensorScale tsr = tensor_scale(gr);
  const float ratio = gr / gx;

  for (int64_t r0 = r_begin; r0 < r_stop; r0 += rb) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    const int nb = nr * cb;
    // a.
    uint2 kc[SLOTS];  // each slot's codes and scale, for X' in c
    uint32_t ksc[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int b = tid + j * kThreads;
      if (j * kThreads < nb && b < nb) {
        kc[j] = raw[j].codes;
        ksc[j] = raw[j].scale;
        if constexpr (kX) {
          const int rr = b / cb;
          store_dx<BF16>(raw[j], gx, region + rr * K, b - rr * cb);
        }
      }
    }
    if (r0 + rb < r_stop) issue(r0 + rb);
    __syncthreads();
    // b.
    for (int t = tid; t < nr * nblk; t += kThreads) {
      const int rr = t / nblk, jb = t - rr * nblk;
      const int64_t row = r0 + rr;
      float *src = region + rr * K;
      // the block's 16 channel offsets, two per word
      const uint4 s0 = reinterpret_cast<const uint4 *>(sel + jb * 16)[0];
      const uint4 s1 = reinterpret_cast<const uint4 *>(sel + jb * 16)[1];
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      auto off = [&](int i) { return static_cast<int>((sw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu); };
      const int nr16 = min(max(n_real - jb * 16, 0), 16);
      const uint32_t real = (1u << nr16) - 1u;  // entries jb*16 + i < n_real
      uint2 rcodes;
      uint32_t rscale;
      if constexpr (kX) {
        float g16[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = src[off(i)];  // pads (offset 0) are zeroed
          g16[i] = (real >> i) & 1u ? v : 0.0f;
        }
        const BlockQ q = quantize_block16(g16, tsr, nullptr);
        rcodes = make_uint2(q.lo, q.hi);
        rscale = q.scale;
        reinterpret_cast<uint2 *>(p.r_codes)[row * nblk + jb] = rcodes;
        p.r_scales[row * nblk + jb] = static_cast<uint8_t>(rscale);
      } else {
        rcodes = reinterpret_cast<const uint2 *>(p.r_codes)[row * nblk + jb];
        rscale = p.r_scales[row * nblk + jb];
      }
      if constexpr (kOut) {
        float rv[16];
        dequant16_signed(rcodes, e4m3_to_f32(rscale), rv);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((real >> i) & 1u) src[off(i)] = rv[i] * ratio;
      }
    }
    if constexpr (kOut) {
      __syncthreads();
      // c.
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) {
        const int b = tid + j * kThreads;
        if (j * kThreads < nb && b < nb) {
          const int cblk = b % cb, c0 = cblk * 16;
          const uint32_t m = (bits[c0 >> 5] >> (c0 & 16)) & 0xFFFFu;
          float cor[16], xv[16];
          const float4 *cp = reinterpret_cast<const float4 *>(region + b * 16);  // row b / cb, block cblk
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = cp[chunk_pos(cblk, q)];
            cor[4 * q] = v.x;
            cor[4 * q + 1] = v.y;
            cor[4 * q + 2] = v.z;
            cor[4 * q + 3] = v.w;
          }
          dequant16_signed(kc[j], e4m3_to_f32(ksc[j]), xv);
          uint4 lo, hi;
          merged_block16(xv, cor, m, lo, hi);
          uint4 *o = reinterpret_cast<uint4 *>(p.merged + (r0 * cb + b) * 16);
          o[0] = lo;
          o[1] = hi;
        }
      }
    }
    if (r0 + rb < r_stop) __syncthreads();  // the rows are rewritten by the next group
  }
}

constexpr size_t kRacLdsTarget = 40 * 1024;  // four workgroups per CU
constexpr size_t kRacLdsMax = 160 * 1024 - 256;
constexpr int kRacMaxRows = 16;

size_t rows_lds_bytes(int64_t cols, int64_t kpad, bool out, int64_t rb) {
  return static_cast<size_t>(kpad * 2 + (out ? bitmap_words(cols) * 4 : 0) + rb * cols * 4);
}

int rows_slots(int64_t cols) { return cols / 16 <= 2 * kThreads ? 2 : kMaxSlots; }

// Dynamic LDS beyond the default limit needs the function attribute.
hipError_t allow_lds(const void *fn, size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

// Row groups and grid of a call: few rows (decode-sized calls) take smaller
// groups, so that the launch still spreads over every CU and each
// workgroup's chain of loads, barriers and stores is short.
int64_t rows_grid(RowsArgs &p) {
  const int64_t spread = (p.rows + 255) / 256;
  if (spread < p.rb) p.rb = static_cast<int>(std::max<int64_t>(1, spread));
  int64_t n_wg = (p.rows + p.rb - 1) / p.rb;
  p.rows_per_wg = p.rb;
  if (n_wg > 1024) {  // about as many workgroups as are resident at once
    p.rows_per_wg = static_cast<int>(p.rb * ((n_wg + 1023) / 1024));
    n_wg = (p.rows + p.rows_per_wg - 1) / p.rows_per_wg;
  }
  return n_wg;
}

template <bool BF16, int MODE, int SLOTS, int MASK_PER>
hipError_t launch_rows_s(const RowsArgs &p, int64_t n_wg, hipStream_t stream) {
  const bool out = MODE != kResidual;
  const size_t lds = rows_lds_bytes(p.K, p.kpad, out, p.rb);
  const hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_rac_rows<BF16, MODE, SLOTS, MASK_PER>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_rac_rows<BF16, MODE, SLOTS, MASK_PER>), dim3(n_wg), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <bool BF16, int MODE>
hipError_t launch_rows_t(RowsArgs p, hipStream_t stream) {
  const int64_t n_wg = rows_grid(p);
  return rows_slots(p.K) == 2 ? launch_rows_s<BF16, MODE, 2, 0>(p, n_wg, stream)
                              : launch_rows_s<BF16, MODE, kMaxSlots, 0>(p, n_wg, stream);
}

template <int PER>
hipError_t launch_mask_t(const RacLaunch &a, hipStream_t stream) {
  hipLaunchKernelGGL((k_rac_mask<PER>), dim3(1), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint32_t *>(a.scores), static_cast<int>(a.cols),
                     static_cast<int>(a.nsel), static_cast<int>(a.kpad), a.sel_idx, a.r_gscale);
  return hipGetLastError();
}

hipError_t launch_mask(const RacLaunch &a, hipStream_t stream) {
  const int64_t per = (a.cols + kThreads - 1) / kThreads;
  if (per <= 4) return launch_mask_t<4>(a, stream);
  if (per <= 8) return launch_mask_t<8>(a, stream);
  if (per <= 16) return launch_mask_t<16>(a, stream);
  if (per <= 32) return launch_mask_t<32>(a, stream);
  return launch_mask_t<64>(a, stream);
}

}  // namespace

int rac_rows_per_group(int64_t cols, int64_t kpad, bool merged) {
  // a row group's blocks fit the per-thread load slots
  int64_t rb = std::min<int64_t>(kRacMaxRows, static_cast<int64_t>(rows_slots(cols)) * kThreads / (cols / 16));
  while (rb > 1 && rows_lds_bytes(cols, kpad, merged, rb) > kRacLdsTarget) --rb;
  if (rb < 1 || rows_lds_bytes(cols, kpad, merged, rb) > kRacLdsMax) return 0;
  return static_cast<int>(rb);
}

hipError_t launch_rac_select(const RacLaunch &a, hipStream_t stream) {
  if (a.cols > 64 * kThreads) return hipErrorInvalidValue;  // the API bounds cols first
  const bool merged = a.merged != nullptr;
  RowsArgs p{};
  p.x = a.x;
  p.rows = a.rows;
  p.K = static_cast<int>(a.cols);
  p.kpad = static_cast<int>(a.kpad);
  p.x_codes = a.x_codes;
  p.x_scales = a.x_scales;
  p.x_g = a.x_gscale;
  p.sel = a.sel_idx;
  p.r_g = a.r_gscale;
  p.r_codes = a.r_codes;
  p.r_scales = a.r_scales;
  p.merged = a.merged;
  p.scores = reinterpret_cast<const uint32_t *>(a.scores);
  p.nsel = static_cast<int>(a.nsel);
  p.sel_out = a.sel_idx;
  p.r_g_out = a.r_gscale;
  p.rb = rac_rows_per_group(a.cols, a.kpad, merged);
  if (a.kpad > 0 && a.rows > 0 && p.rb < 1) return hipErrorInvalidValue;
  // bf16 rows of up to 2048 channels, in calls of at most one workgroup per
  // CU or with at least 8 row groups per workgroup: each workgroup finds the
  // mask itself (one launch).  Measured: decode x 11.5 -> 8.9 us, prefill h
  // 117 -> 113 us; with one row group per workgroup and four workgroups per
  // CU (4096 x 2048) the separate mask launch is faster (20.2 against 22.8 us).
  if (a.kpad > 0 && a.rows > 0 && a.x_bf16 && a.cols <= 2 * kThreads * 4) {
    RowsArgs q = p;
    const int64_t n_wg = rows_grid(q);
    if ((n_wg <= 256 || q.rows_per_wg >= 8 * q.rb) && rows_slots(q.K) == 2) {
      if (a.cols <= 4 * kThreads)
        return merged ? launch_rows_s<true, kMerged, 2, 4>(q, n_wg, stream)
                      : launch_rows_s<true, kResidual, 2, 4>(q, n_wg, stream);
      return merged ? launch_rows_s<true, kMerged, 2, 8>(q, n_wg, stream)
                    : launch_rows_s<true, kResidual, 2, 8>(q, n_wg, stream);
    }
  }
  const hipError_t e = launch_mask(a, stream);
  if (e != hipSuccess || a.kpad == 0 || a.rows == 0) return e;
  if (a.x_bf16)
    return merged ? launch_rows_t<true, kMerged>(p, stream) : launch_rows_t<true, kResidual>(p, stream);
  return merged ? launch_rows_t<false, kMerged>(p, stream) : launch_rows_t<false, kResidual>(p, stream);
}

hipError_t launch_rac_merge_codes(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_g,
                                  const uint8_t *r_codes, const uint8_t *r_scales, const float *r_g, int64_t rows,
                                  int64_t cols, int64_t kpad, const int32_t *sel_idx, uint16_t *merged,
                                  hipStream_t stream) {
  if (kpad == 0 || rows == 0) return hipSuccess;
  RowsArgs p{};
  p.rows = rows;
  p.K = static_cast<int>(cols);
  p.kpad = static_cast<int>(kpad);
  p.x_codes = x_codes;
  p.x_scales = x_scales;
  p.x_g = x_g;
  p.sel = sel_idx;
  p.r_g = r_g;
  p.r_codes = const_cast<uint8_t *>(r_codes);  // read only in this mode
  p.r_scales = const_cast<uint8_t *>(r_scales);
  p.merged = merged;
  p.rb = rac_rows_per_group(cols, kpad, true);
  if (p.rb < 1) return hipErrorInvalidValue;
  return launch_rows_t<true, kFromCodes>(p, stream);
}

}  // namespace quads
