// Residual Activation Compensation (RAC) on gfx950: channel mask and
// second-pass residual quantization.
//
// QUADS technical summary, section 2.2-B: channels whose first-pass FP4
// residual is largest get a binary mask (the top k% of channels, 50% being the
// example setting) and their residual is quantized a second time; that
// correction is added to the quantized path, so the native W4A4 GEMM still
// does most of the work.
//
//   k_rac_select    one 1024-thread workgroup: radix select (4 passes of 8
//                   bits over the FP32 score bit patterns, which order like
//                   the non-negative floats they encode) finds the nsel-th
//                   largest score T; channels above T plus the lowest-index
//                   channels equal to T are kept; a block-wide prefix sum
//                   writes them in ascending order.  Also writes the residual
//                   tensor scale from the largest score.
//   k_rac_residual  stages rows of x, their codes and scales in LDS, recomputes
//                   dx = x - dq at the selected channels (same FP32 operations
//                   as the quantizer) and NVFP4-quantizes the gathered
//                   residual in 16-element blocks along the selected order.
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kMaxSelCols = 16384;

// Exclusive prefix sum over the 1024 threads of the block; returns the
// exclusive prefix of `v` and stores the block total in *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wave_sums,
                                                         uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  __syncthreads();
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      const uint32_t s = wave_sums[w];
      wave_sums[w] = run;
      run += s;
    }
    wave_sums[kSelThreads / 64] = run;
  }
  __syncthreads();
  *total = wave_sums[kSelThreads / 64];
  return wave_sums[wave] + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void k_rac_select(const uint32_t *scores, int K, int nsel,
                                                            int kpad, int32_t *sel, float *res_g) {
  __shared__ uint32_t keys[kMaxSelCols];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_sums[kSelThreads / 64 + 1];
  __shared__ uint32_t s_prefix, s_remaining, s_max;
  const int tid = threadIdx.x;
  if (tid == 0) s_max = 0;
  __syncthreads();
  uint32_t mymax = 0;
  for (int c = tid; c < K; c += kSelThreads) {
    const uint32_t k = scores[c];
    keys[c] = k;
    mymax = max(mymax, k);
  }
  atomicMax(&s_max, mymax);  // LDS atomic
  __syncthreads();
  if (tid == 0) *res_g = tensor_scale_from_amax(nsel > 0 ? __uint_as_float(s_max) : 0.0f);
  for (int j = nsel + tid; j < kpad; j += kSelThreads) sel[j] = 0;
  if (nsel == 0) return;

  // Radix select of the nsel-th largest key.
  if (tid == 0) {
    s_prefix = 0;
    s_remaining = static_cast<uint32_t>(nsel);
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int c = tid; c < K; c += kSelThreads) {
      const uint32_t k = keys[c];
      const bool match = shift == 24 || ((k ^ prefix) >> (shift + 8)) == 0;
      if (match) atomicAdd(&hist[(k >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // Suffix counts over bins, 4 bins per lane, highest bins first.
      const int lane = tid;
      uint32_t c4[4];
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c4[q] = hist[255 - (lane * 4 + q)];
        sum += c4[q];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      uint32_t before = incl - sum;  // keys in bins above this lane's first bin
      const uint32_t need = s_remaining;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (before < need && before + c4[q] >= need) {
          const uint32_t bin = 255u - static_cast<uint32_t>(lane * 4 + q);
          s_prefix = prefix | (bin << shift);
          s_remaining = need - before;
        }
        before += c4[q];
      }
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const uint32_t need_eq = s_remaining;  // how many keys equal to T are kept

  // Each thread owns a contiguous run of channels (keeps ascending order).
  const int per = (K + kSelThreads - 1) / kSelThreads;
  const int c0 = tid * per, c1 = min(c0 + per, K);
  uint32_t n_eq = 0;
  for (int c = c0; c < c1; ++c) n_eq += keys[c] == T;
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(n_eq, wave_sums, &tot);
  uint32_t n_keep = 0;
  {
    uint32_t e = eq_before;
    for (int c = c0; c < c1; ++c) {
      const uint32_t k = keys[c];
      if (k > T) {
        ++n_keep;
      } else if (k == T) {
        n_keep += e < need_eq;
        ++e;
      }
    }
  }
  uint32_t pos = block_exclusive_scan(n_keep, wave_sums, &tot);
  {
    uint32_t e = eq_before;
    for (int c = c0; c < c1; ++c) {
      const uint32_t k = keys[c];
      bool keep = false;
      if (k > T) {
        keep = true;
      } else if (k == T) {
        keep = e < need_eq;
        ++e;
      }
      if (keep) sel[pos++] = c;
    }
  }
}

// Residual quantization.  One workgroup handles `rb` rows at a time: x, codes
// and scales of those rows are staged in LDS with 16-byte loads, then each
// thread quantizes 16-element residual blocks (row, j-block) from LDS.
// row_bytes = x bytes + cols/2 + cols/16, rounded up to 16.
template <bool BF16>
__global__ __launch_bounds__(256) void k_rac_residual(const void *x, int64_t rows, int cols,
                                                      const uint8_t *x_codes,
                                                      const uint8_t *x_scales, const float *x_g,
                                                      const int32_t *sel, int nsel, int kpad,
                                                      const float *r_g, uint8_t *r_codes,
                                                      uint8_t *r_scales, int rb, int rows_per_wg,
                                                      int row_bytes) {
  extern __shared__ uint4 lds_u4[];
  uint8_t *lds = reinterpret_cast<uint8_t *>(lds_u4);
  const int xbytes = cols * (BF16 ? 2 : 4);  // multiple of 32
  const int cbytes = cols / 2;                // multiple of 8
  const int sbytes = cols / 16;
  int32_t *sel_l = reinterpret_cast<int32_t *>(lds);
  uint8_t *rows_l = lds + static_cast<size_t>(kpad) * 4;
  for (int j = threadIdx.x; j < kpad; j += 256) sel_l[j] = j < nsel ? sel[j] : -1;
  const float gx = *x_g, gr = *r_g;
  const int nblk = kpad / 16;
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t r_stop = min(r_begin + rows_per_wg, rows);
  for (int64_t r0 = r_begin; r0 < r_stop; r0 += rb) {
    const int nr = static_cast<int>(min(static_cast<int64_t>(rb), r_stop - r0));
    __syncthreads();
    // x rows are contiguous in global memory: one flat 16-byte copy per row set.
    {
      const int xv = xbytes / 16;
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + r0 * xbytes);
      for (int i = threadIdx.x; i < nr * xv; i += 256) {
        const int rr = i / xv, c = i % xv;
        reinterpret_cast<uint4 *>(rows_l + static_cast<size_t>(rr) * row_bytes)[c] = src[i];
      }
    }
    {
      const int cv = cbytes / 8;
      const uint2 *src = reinterpret_cast<const uint2 *>(x_codes + r0 * cbytes);
      for (int i = threadIdx.x; i < nr * cv; i += 256) {
        const int rr = i / cv, c = i % cv;
        reinterpret_cast<uint2 *>(rows_l + static_cast<size_t>(rr) * row_bytes + xbytes)[c] = src[i];
      }
    }
    {
      const uint8_t *src = x_scales + r0 * sbytes;
      for (int i = threadIdx.x; i < nr * sbytes; i += 256) {
        const int rr = i / sbytes, c = i % sbytes;
        rows_l[static_cast<size_t>(rr) * row_bytes + xbytes + cbytes + c] = src[i];
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < nr * nblk; t += 256) {
      const int rr = t / nblk, jb = t % nblk;
      const uint8_t *rowp = rows_l + static_cast<size_t>(rr) * row_bytes;
      float d16[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = sel_l[jb * 16 + i];
        float dx = 0.0f;
        if (c >= 0) {
          float xv;
          if constexpr (BF16)
            xv = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(rowp)[c]);
          else
            xv = reinterpret_cast<const float *>(rowp)[c];
          const uint32_t code = (rowp[xbytes + (c >> 1)] >> ((c & 1) * 4)) & 0xFu;
          const float d = e4m3_to_f32(rowp[xbytes + cbytes + (c >> 4)]) * gx;
          dx = xv - dequant_code(code, d);
        }
        d16[i] = dx;
      }
      const BlockQ q = quantize_block16(d16, gr, nullptr);
      const int64_t row = r0 + rr;
      reinterpret_cast<uint2 *>(r_codes)[row * nblk + jb] = make_uint2(q.lo, q.hi);
      r_scales[row * nblk + jb] = static_cast<uint8_t>(q.scale);
    }
  }
}

}  // namespace

hipError_t launch_rac_select(const RacLaunch &a, hipStream_t stream) {
  hipLaunchKernelGGL(k_rac_select, dim3(1), dim3(kSelThreads), 0, stream,
                     reinterpret_cast<const uint32_t *>(a.scores), static_cast<int>(a.cols),
                     static_cast<int>(a.nsel), static_cast<int>(a.kpad), a.sel_idx, a.r_gscale);
  if (a.kpad == 0 || a.rows == 0) return hipGetLastError();
  const int cols = static_cast<int>(a.cols);
  const int row_bytes = (cols * (a.x_bf16 ? 2 : 4) + cols / 2 + cols / 16 + 15) / 16 * 16;
  const int budget = 64 * 1024 - static_cast<int>(a.kpad) * 4;
  int rb = budget / row_bytes;
  if (rb > 16) rb = 16;
  if (rb < 1) rb = 1;
  int64_t n_wg = (a.rows + rb - 1) / rb;
  int rows_per_wg = rb;
  if (n_wg > 1024) {
    const int64_t iters = (n_wg + 1023) / 1024;
    rows_per_wg = static_cast<int>(rb * iters);
    n_wg = (a.rows + rows_per_wg - 1) / rows_per_wg;
  }
  const size_t lds = static_cast<size_t>(a.kpad) * 4 + static_cast<size_t>(rb) * row_bytes;
  if (a.x_bf16)
    hipLaunchKernelGGL(k_rac_residual<true>, dim3(n_wg), dim3(256), lds, stream, a.x, a.rows, cols,
                       a.x_codes, a.x_scales, a.x_gscale, a.sel_idx, static_cast<int>(a.nsel),
                       static_cast<int>(a.kpad), a.r_gscale, a.r_codes, a.r_scales, rb, rows_per_wg,
                       row_bytes);
  else
    hipLaunchKernelGGL(k_rac_residual<false>, dim3(n_wg), dim3(256), lds, stream, a.x, a.rows, cols,
                       a.x_codes, a.x_scales, a.x_gscale, a.sel_idx, static_cast<int>(a.nsel),
                       static_cast<int>(a.kpad), a.r_gscale, a.r_codes, a.r_scales, rb, rows_per_wg,
                       row_bytes);
  return hipGetLastError();
}

}  // namespace quads
