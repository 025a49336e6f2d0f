// NVFP4 quantization kernels (activation quantize + RAC channel scores, and
// the trainer weight QDQ), gfx950.
//
// The activation quantization is what the QUADS technical summary
// (section 2.1) describes as recomputed online on every rollout forward; the
// channel score (max over rows of the first-pass residual |x - dq|) is what
// RAC (section 2.2-B) ranks channels by; the QDQ output (bf16 of dq) is the
// trainer's fake-quantized weight (section 2.2-A).
//
// Two launches per call, no atomics on floats and no memset:
//   k_amax_partial  one max|x| partial per workgroup (P per tensor), over
//                   contiguous chunks (weight batches) or, for one activation
//                   matrix, over k_quantize's own tiles (k_amax_tiles); also
//                   zeroes the score buffer when scores are requested;
//   k_quantize      every workgroup folds its tensor's P partials into g, then
//                   quantizes a [rows x 16*BC] tile: 16-element blocks,
//                   one block per thread per row step, coalesced 32/64-byte
//                   loads, 8-byte code stores, optional bf16 QDQ stores, and a
//                   per-workgroup column max of |x - dq| merged with one u32
//                   atomicMax per column (order-independent, so deterministic).
#include <mutex>

#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kThreads = 256;

// 16 elements as loaded (bf16: 2 x 16 bytes, fp32: 4 x 16 bytes); converted
// to FP32 only where they are used, so a load can be issued early.
template <bool BF16>
struct Raw16 {
  uint4 u[BF16 ? 2 : 4];
};

// NT: nontemporal loads (weights, read once); plain loads keep an
// activation in L2 for the pass that reads it next.
template <bool BF16, bool NT>
__device__ __forceinline__ void load_raw16(const void *base, int64_t elem, Raw16<BF16> &r) {
  const uint4 *p = BF16 ? reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem)
                        : reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + elem);
#pragma unroll
  for (int i = 0; i < (BF16 ? 2 : 4); ++i) r.u[i] = NT ? load_nt16(p + i) : p[i];
}

template <bool BF16>
__device__ __forceinline__ void to_f32(const Raw16<BF16> &r, float (&v)[16]) {
  if constexpr (BF16) {
    const uint32_t w[8] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w, r.u[1].x, r.u[1].y, r.u[1].z, r.u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = __uint_as_float(r.u[i].x);
      v[4 * i + 1] = __uint_as_float(r.u[i].y);
      v[4 * i + 2] = __uint_as_float(r.u[i].z);
      v[4 * i + 3] = __uint_as_float(r.u[i].w);
    }
  }
}

// Max over the wave of non-negative floats (amax values), on their bit
// patterns, which order like the values.
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(last_lane(wave_scan<true>(__float_as_uint(v))));
}

// Block-wide max of non-negative floats over kThreads threads; result valid
// in every thread.
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <bool BF16, bool NT = true>
__global__ __launch_bounds__(kThreads) void k_amax_partial(const void *x, int64_t n_per_tensor,
                                                           int P, int64_t chunk, float *partials,
                                                           float *scores, int64_t cols) {
  __shared__ float red[kThreads / 64];
  const int b = blockIdx.x / P, p = blockIdx.x % P;
  const int64_t start = p * chunk;
  const int64_t end = min(start + chunk, n_per_tensor);
  const int64_t base = static_cast<int64_t>(b) * n_per_tensor;
  float m = 0.0f;
  constexpr int kVec = BF16 ? 8 : 4;  // elements per 16-byte load
  constexpr int kUnroll = 4;          // loads in flight per thread
  const int64_t stride = static_cast<int64_t>(kThreads) * kVec;
  auto fold = [&](const uint4 &u) {
    if constexpr (BF16) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = fmaxf(m, fabsf(__uint_as_float(w[k] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(w[k] & 0xFFFF0000u)));
      }
    } else {
      m = fmaxf(fmaxf(fabsf(__uint_as_float(u.x)), fabsf(__uint_as_float(u.y))),
                fmaxf(fmaxf(fabsf(__uint_as_float(u.z)), fabsf(__uint_as_float(u.w))), m));
    }
  };
  auto addr = [&](int64_t i) -> const void * {
    if constexpr (BF16) return static_cast<const uint16_t *>(x) + base + i;
    else return static_cast<const float *>(x) + base + i;
  };
  int64_t i = start + static_cast<int64_t>(threadIdx.x) * kVec;
  for (; i + (kUnroll - 1) * stride < end; i += kUnroll * stride) {
    uint4 u[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      u[k] = NT ? load_nt16(addr(i + k * stride)) : *reinterpret_cast<const uint4 *>(addr(i + k * stride));
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) fold(u[k]);
  }
  for (; i < end; i += stride) fold(NT ? load_nt16(addr(i)) : *reinterpret_cast<const uint4 *>(addr(i)));
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
  if (scores != nullptr && blockIdx.x == 0) {
    for (int64_t c = threadIdx.x; c < cols; c += kThreads) scores[c] = 0.0f;
  }
}

// Tensor scale of matrix blockIdx.x from its P amax partials (the fold
// k_quantize does for its own tensor).
__global__ __launch_bounds__(kThreads) void k_fold_gscale(const float *partials, int P, float *gscale) {
  __shared__ float red[kThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < P; i += kThreads) m = fmaxf(m, partials[static_cast<int64_t>(blockIdx.x) * P + i]);
  const float g = tensor_scale_from_amax(block_max(m, red));
  if (threadIdx.x == 0) gscale[blockIdx.x] = g;
}

__global__ __launch_bounds__(kThreads) void k_fill_one(float *p, int64_t n) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x;
  if (i < n) p[i] = 1.0f;
}

__global__ __launch_bounds__(kThreads) void k_zero_f32(float *p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    p[i] = 0.0f;
}

// An activation with no rows: the largest of no magnitudes is taken as 0, so
// the tensor scale is 1 (the all-zero convention) and every channel score 0.
__global__ __launch_bounds__(kThreads) void k_empty_tensor(float *gscale, int64_t batch, float *scores, int64_t cols) {
  if (gscale != nullptr)
    for (int64_t b = threadIdx.x; b < batch; b += kThreads) gscale[b] = 1.0f;
  if (scores != nullptr)
    for (int64_t c = threadIdx.x; c < cols; c += kThreads) scores[c] = 0.0f;
}

struct QParams {
  const void *x;
  int64_t rows, cols, cb;  // cb = cols / 16
  int BC, RG, RW;          // blocks per row step, rows per step, rows per workgroup
  int col_chunks, row_chunks, P;
  const float *partials;
  float *gscale;
  int gscale_given;
  uint8_t *codes, *scales;
  float *scores;
  uint16_t *qdq;
};

template <bool BF16, bool SCORES, bool CODES, bool QDQ, bool NT>
__global__ __launch_bounds__(kThreads) void k_quantize(QParams p) {
  __shared__ float red[kThreads / 64];
  extern __shared__ float smax_lds[];  // [RG][BC*16] when SCORES
  const int per_tensor = p.row_chunks * p.col_chunks;
  const int b = blockIdx.x / per_tensor;
  const int rem = blockIdx.x % per_tensor;
  const int rc = rem / p.col_chunks, cc = rem % p.col_chunks;

  const int bcol = threadIdx.x % p.BC, rg = threadIdx.x / p.BC;
  const int64_t gbc = static_cast<int64_t>(cc) * p.BC + bcol;
  const bool active = rg < p.RG && gbc < p.cb;
  const int64_t r_end = min(static_cast<int64_t>(rc + 1) * p.RW, p.rows);
  int64_t r = static_cast<int64_t>(rc) * p.RW + rg;

  // Rows are taken in pairs (r, r + RG); the next pair's loads are in
  // flight while the current pair is quantized.
  struct Pair {
    Raw16<BF16> x[2];
    int64_t row[2];
    bool two;
  };
  Pair pa, pb;
  auto issue = [&](Pair &q, int64_t rr) {
    q.two = rr + p.RG < r_end;
    q.row[0] = static_cast<int64_t>(b) * p.rows + rr;
    q.row[1] = q.row[0] + (q.two ? p.RG : 0);
    load_raw16<BF16, NT>(p.x, q.row[0] * p.cols + gbc * 16, q.x[0]);
    load_raw16<BF16, NT>(p.x, q.row[1] * p.cols + gbc * 16, q.x[1]);
  };
  if (active && r < r_end) issue(pa, r);  // in flight while the tensor scale is folded

  float g;
  if (p.gscale_given) {
    g = p.gscale[b];
  } else {
    float m = 0.0f;
    for (int i = threadIdx.x; i < p.P; i += kThreads) m = fmaxf(m, p.partials[b * p.P + i]);
    g = tensor_scale_from_amax(block_max(m, red));
    if (p.gscale != nullptr && rc == 0 && cc == 0 && threadIdx.x == 0) p.gscale[b] = g;
  }
  const TensorScale ts = tensor_scale(g);

  float smax[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) smax[i] = 0.0f;

  auto quantize_pair = [&](const Pair &q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !q.two) break;
      const int64_t row = q.row[u];
      float v[16];
      to_f32<BF16>(q.x[u], v);
      float dq[16];
      const BlockQ bq = quantize_block16(v, ts, (SCORES || QDQ) ? dq : nullptr);
      if constexpr (CODES) {
        reinterpret_cast<uint2 *>(p.codes)[row * p.cb + gbc] = make_uint2(bq.lo, bq.hi);
        p.scales[row * p.cb + gbc] = static_cast<uint8_t>(bq.scale);
      }
      if constexpr (QDQ) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(dq[2 * i], dq[2 * i + 1]);
        uint4 *o = reinterpret_cast<uint4 *>(p.qdq + row * p.cols + gbc * 16);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
      if constexpr (SCORES) {
#pragma unroll
        for (int i = 0; i < 16; ++i) smax[i] = fmaxf(smax[i], fabsf(v[i] - dq[i]));
      }
    }
  };
  if (active && r < r_end) {
    for (;;) {
      const int64_t r1 = r + 2 * p.RG;
      if (r1 < r_end) issue(pb, r1);
      quantize_pair(pa);
      if (r1 >= r_end) break;
      const int64_t r2 = r1 + 2 * p.RG;
      if (r2 < r_end) issue(pa, r2);
      quantize_pair(pb);
      if (r2 >= r_end) break;
      r = r2;
    }
  }

  if constexpr (SCORES) {
    const int width = p.BC * 16;
    if (rg < p.RG) {
#pragma unroll
      for (int i = 0; i < 16; ++i) smax_lds[rg * width + bcol * 16 + i] = smax[i];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < width; c += kThreads) {
      float m = 0.0f;
      for (int k = 0; k < p.RG; ++k) m = fmaxf(m, smax_lds[k * width + c]);
      const int64_t gc = static_cast<int64_t>(cc) * width + c;
      if (gc < p.cols && m > 0.0f)
        atomicMax(reinterpret_cast<unsigned int *>(p.scores) + gc, __float_as_uint(m));
    }
  }
}

// The amax pass of one activation matrix over the quantizer's own tiles:
// workgroup w folds tiles w, w + P, ... (the (row chunk, column chunk) tiles
// k_quantize numbers the same way) into partial w, with plain loads.  With P
// a multiple of 8 (4096 x 2048 with scores: 512 tiles and partials), each
// tile is read by workgroups of the same index, on the same XCD, in both
// passes.  Plain instead of nontemporal loads in both passes gave most of the
// gain (expert-GEMM step 72.8 -> 71.0 us, prefill quantize of h 60 -> 54 us;
// the quantizer's counted HBM-side fetch stays at 1.06x, so the second read
// is served beyond L2), the tiled amax pass another 0.7 us (70.3 us).
// Weight batches keep the contiguous-chunk pass and nontemporal loads (590
// against 744 us per gate_up QDQ the other way).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_amax_tiles(QParams p, float *partials) {
  __shared__ float red[kThreads / 64];
  const int per_tensor = p.row_chunks * p.col_chunks;
  const int b = blockIdx.x / p.P, w = blockIdx.x % p.P;
  const int bcol = threadIdx.x % p.BC, rg = threadIdx.x / p.BC;
  float m = 0.0f;
  for (int t = w; t < per_tensor; t += p.P) {
    const int rc = t / p.col_chunks, cc = t % p.col_chunks;
    const int64_t gbc = static_cast<int64_t>(cc) * p.BC + bcol;
    if (rg >= p.RG || gbc >= p.cb) continue;
    const int64_t r_end = min(static_cast<int64_t>(rc + 1) * p.RW, p.rows);
    for (int64_t r = static_cast<int64_t>(rc) * p.RW + rg; r < r_end; r += p.RG) {
      const int64_t elem = (static_cast<int64_t>(b) * p.rows + r) * p.cols + gbc * 16;
      Raw16<BF16> raw;
      load_raw16<BF16, false>(p.x, elem, raw);
      float v[16];
      to_f32<BF16>(raw, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
  if (p.scores != nullptr && blockIdx.x == 0)
    for (int64_t c = threadIdx.x; c < p.cols; c += kThreads) p.scores[c] = 0.0f;
}

template <bool BF16, bool SCORES, bool CODES, bool QDQ, bool NT>
void launch_q(const QParams &qp, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_quantize<BF16, SCORES, CODES, QDQ, NT>), dim3(grid), dim3(kThreads), lds, s, qp);
}

}  // namespace

int amax_partials_per_tensor(int64_t n_elem) {
  int64_t p = (n_elem + 16383) / 16384;
  if (p < 1) p = 1;
  if (p > 1024) p = 1024;
  return static_cast<int>(p);
}

size_t quantize_ws_bytes(int64_t batch, int64_t rows, int64_t cols) {
  const int P = amax_partials_per_tensor(rows * cols);
  return static_cast<size_t>(batch) * P * sizeof(float) + 256;
}

hipError_t launch_tensor_scales(const void *x, bool x_bf16, int64_t batch, int64_t rows, int64_t cols, float *gscale,
                                void *ws, hipStream_t stream) {
  const int64_t n = rows * cols;
  const int P = amax_partials_per_tensor(n);
  float *partials = static_cast<float *>(ws);
  if (n == 0) {
    hipLaunchKernelGGL(k_fill_one, dim3((batch + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, gscale, batch);
    return hipGetLastError();
  }
  int64_t chunk = (n + P - 1) / P;
  chunk = (chunk + 15) / 16 * 16;
  if (x_bf16)
    hipLaunchKernelGGL(k_amax_partial<true>, dim3(batch * P), dim3(kThreads), 0, stream, x, n, P, chunk, partials,
                       nullptr, cols);
  else
    hipLaunchKernelGGL(k_amax_partial<false>, dim3(batch * P), dim3(kThreads), 0, stream, x, n, P, chunk, partials,
                       nullptr, cols);
  hipLaunchKernelGGL(k_fold_gscale, dim3(batch), dim3(kThreads), 0, stream, partials, P, gscale);
  return hipGetLastError();
}

size_t quantize_partials_bytes(int64_t batch, int64_t rows, int64_t cols) {
  return static_cast<size_t>(batch) * amax_partials_per_tensor(rows * cols) * sizeof(float);
}

// The amax partials of quads_quantize_nvfp4_noalloc live in this file-scope
// device array instead of a caller workspace: one copy per GPU the library
// runs on, held until the process ends, shared by every such call on that
// GPU (each call writes every partial it reads, so nothing needs clearing).
// Host code never uses the array's name as an address: its device address is
// looked up once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t quantize_scratch(float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float *>(g_scratch_ptr[dev]);
  return hipSuccess;
}

hipError_t launch_quantize(const QuantizeLaunch &a, hipStream_t stream) {
  if (a.rows == 0) {  // nothing to quantize: the tensor scales (unless given) and the scores
    if (a.gscale_given && a.scores == nullptr) return hipSuccess;
    hipLaunchKernelGGL(k_empty_tensor, dim3(1), dim3(kThreads), 0, stream, a.gscale_given ? nullptr : a.gscale,
                       a.batch, a.scores, a.cols);
    return hipGetLastError();
  }
  const int64_t n = a.rows * a.cols;
  const int P = amax_partials_per_tensor(n);
  float *partials = static_cast<float *>(a.ws);

  QParams qp{};
  qp.x = a.x;
  qp.rows = a.rows;
  qp.cols = a.cols;
  qp.cb = a.cols / 16;
  // With channel scores, tiles of 16 blocks (256 channels, 16 rows per step):
  // each row's codes leave as one whole 128-byte line (narrower tiles left
  // partial lines shared between workgroups: 1.8x the written bytes), at 256
  // column-max atomics per workgroup and about 1024 workgroups.  Measured on
  // 4096 x 2048 bf16, amax pass included: 4 blocks 16.6 us, 8 blocks 15.3 us,
  // 16 blocks 14.9 us, 32 blocks 16.0 us.
  const int64_t bc_max = a.scores != nullptr ? 16 : 64;
  qp.BC = static_cast<int>(qp.cb < bc_max ? qp.cb : bc_max);
  qp.RG = kThreads / qp.BC;
  qp.col_chunks = static_cast<int>((qp.cb + qp.BC - 1) / qp.BC);
  const int64_t steps = a.batch * ((a.rows + qp.RG - 1) / qp.RG) * qp.col_chunks;
  // About 1024 workgroups, but at least 4 row steps (two pipelined pairs) per
  // workgroup while that still leaves 512 of them (4096 x 2048 bf16 with
  // scores: 15.3 -> 13.9 us per call).
  int64_t iters = steps / 1024;
  if (iters < 4) iters = steps / 512 < 4 ? steps / 512 : 4;
  if (iters < 1) iters = 1;
  if (iters > 64) iters = 64;
  qp.RW = static_cast<int>(qp.RG * iters);
  qp.row_chunks = static_cast<int>((a.rows + qp.RW - 1) / qp.RW);
  qp.P = P;
  qp.partials = partials;
  qp.gscale = a.gscale;
  qp.gscale_given = a.gscale_given ? 1 : 0;
  qp.codes = a.codes;
  qp.scales = a.scales;
  qp.scores = a.scores;
  qp.qdq = a.qdq_out;
  // One matrix (an activation, read again by the quantize pass and by RAC):
  // plain loads in both passes, and the amax over the quantizer's tiles where
  // they map onto the partials (at most two tiles per partial, P a multiple
  // of 8; decode-sized calls, whose few partials would each fold many tiles,
  // measured 0.8 us slower that way and keep contiguous chunks).  Weight
  // batches (read once): contiguous chunks and nontemporal loads.
  const int64_t tiles = static_cast<int64_t>(qp.row_chunks) * qp.col_chunks;
  const bool act = a.batch == 1;  // plain loads
  const bool tiled = act && P % 8 == 0 && tiles <= 2 * static_cast<int64_t>(P);
  if (!a.gscale_given) {
    if (tiled) {
      if (a.x_bf16) hipLaunchKernelGGL(k_amax_tiles<true>, dim3(P), dim3(kThreads), 0, stream, qp, partials);
      else hipLaunchKernelGGL(k_amax_tiles<false>, dim3(P), dim3(kThreads), 0, stream, qp, partials);
    } else {
      int64_t chunk = (n + P - 1) / P;
      chunk = (chunk + 15) / 16 * 16;
      if (a.x_bf16 && act)
        hipLaunchKernelGGL((k_amax_partial<true, false>), dim3(P), dim3(kThreads), 0, stream, a.x, n, P, chunk,
                           partials, a.scores, a.cols);
      else if (a.x_bf16)
        hipLaunchKernelGGL((k_amax_partial<true, true>), dim3(a.batch * P), dim3(kThreads), 0, stream, a.x, n, P,
                           chunk, partials, a.scores, a.cols);
      else if (act)
        hipLaunchKernelGGL((k_amax_partial<false, false>), dim3(P), dim3(kThreads), 0, stream, a.x, n, P, chunk,
                           partials, a.scores, a.cols);
      else
        hipLaunchKernelGGL((k_amax_partial<false, true>), dim3(a.batch * P), dim3(kThreads), 0, stream, a.x, n, P,
                           chunk, partials, a.scores, a.cols);
    }
  } else if (a.scores != nullptr) {
    hipLaunchKernelGGL(k_zero_f32, dim3(1), dim3(kThreads), 0, stream, a.scores, a.cols);
  }
  const int grid = static_cast<int>(a.batch * qp.row_chunks * qp.col_chunks);
  const bool scores = a.scores != nullptr, codes = a.codes != nullptr, qdq = a.qdq_out != nullptr;
  const size_t lds = scores ? static_cast<size_t>(qp.RG) * qp.BC * 16 * sizeof(float) : 0;
  if (a.x_bf16) {
    if (scores && act)  // (scores: batch 1)
      launch_q<true, true, true, false, false>(qp, grid, lds, stream);
    else if (scores)
      launch_q<true, true, true, false, true>(qp, grid, lds, stream);
    else if (codes && qdq)
      launch_q<true, false, true, true, true>(qp, grid, lds, stream);
    else if (qdq)
      launch_q<true, false, false, true, true>(qp, grid, lds, stream);
    else if (act)
      launch_q<true, false, true, false, false>(qp, grid, lds, stream);
    else
      launch_q<true, false, true, false, true>(qp, grid, lds, stream);
  } else {
    if (scores && act)
      launch_q<false, true, true, false, false>(qp, grid, lds, stream);
    else if (scores)
      launch_q<false, true, true, false, true>(qp, grid, lds, stream);
    else if (codes && qdq)
      launch_q<false, false, true, true, true>(qp, grid, lds, stream);
    else if (qdq)
      launch_q<false, false, false, true, true>(qp, grid, lds, stream);
    else if (act)
      launch_q<false, false, true, false, false>(qp, grid, lds, stream);
    else
      launch_q<false, false, true, false, true>(qp, grid, lds, stream);
  }
  return hipGetLastError();
}

}  // namespace quads
