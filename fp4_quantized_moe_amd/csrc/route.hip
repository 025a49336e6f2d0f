// MoE support steps around the expert GEMM on gfx950: top-k softmax routing,
// the (expert, token)-ordered permutation of routed rows, and the combine.
// The pages describe experts and expert-grouped execution, not the routing
// mechanics; this is standard top-k softmax routing with deterministic ties.
//
//   k_route_topk     one wave per token: softmax statistics and top-k by
//                    repeated wave argmax (ties to the lower expert index);
//                    for E <= 256 k_route_topk_rank gives the same top-k by
//                    ranking every logit against the token's others in LDS
//   k_route_count    per 256-token block, per-expert counts (LDS atomics on
//                    integers: exact and order-independent)
//   k_route_scan     block offsets per expert and expert_offsets[E+1]
//   k_route_scatter  rank of a token among the block's tokens that chose the
//                    same expert (popcount over an LDS bitmap), giving
//                    row_token and inverse without any ordering race
//   k_route_one_block  the last three in one workgroup when T <= 256
//   k_combine        out[t] = sum over slots (in order) of w * y[row]
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int kTokBlk = 256;

// Selection key of a logit: an unsigned integer that orders like the value,
// with -0 equal to +0 and NaN below -inf (key 0; -inf is 0x007FFFFF).  Both
// top-k kernels pick experts by (key descending, index ascending), so every
// written id is a valid expert whatever the logits hold, and a NaN logit is
// chosen only after every real one (-inf included), as a stable descending
// sort puts it.
__device__ __forceinline__ uint32_t route_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (v != v) return 0u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave-wide maximum of a 64-bit value with DPP moves (the row shifts and row
// broadcasts of wave_scan): no LDS round trip per level, as a shuffle has.
// Lanes whose DPP source lies outside the row take 0, the identity here.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_max64_step(uint32_t &hi, uint32_t &lo) {
  const uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(hi), CTRL, ROW_MASK, 0xf, false));
  const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(lo), CTRL, ROW_MASK, 0xf, false));
  if (h > hi || (h == hi && l > lo)) {
    hi = h;
    lo = l;
  }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t hi = static_cast<uint32_t>(v >> 32), lo = static_cast<uint32_t>(v);
  dpp_max64_step<0x111, 0xf>(hi, lo);
  dpp_max64_step<0x112, 0xf>(hi, lo);
  dpp_max64_step<0x114, 0xf>(hi, lo);
  dpp_max64_step<0x118, 0xf>(hi, lo);
  dpp_max64_step<0x142, 0xa>(hi, lo);
  dpp_max64_step<0x143, 0xc>(hi, lo);
  return (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), 63))) << 32) |
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), 63));
}

// kMaxPer = ceil(E / 64) slots per lane (E <= 64 * kMaxPer <= 1024).
template <int kMaxPer>
__global__ __launch_bounds__(256) void k_route_topk(const float *logits, int64_t T, int E, int top,
                                                    int32_t *ids, float *wts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + t * E;
  float v[kMaxPer];
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) {
    const int e = q * 64 + lane;
    v[q] = e < E ? row[e] : -INFINITY;
    mx = fmaxf(mx, v[q]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q)
    if (q * 64 + lane < E) sum += expf(v[q] - mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  uint32_t key[kMaxPer];
#pragma unroll
  for (int q = 0; q < kMaxPer; ++q) key[q] = route_key(v[q]);
  uint32_t taken = 0;  // bit q: slot q of this lane already chosen
  for (int j = 0; j < top; ++j) {
    // Each lane's best untaken expert packed as key << 32 | (2^32 - 1 - e),
    // so that the larger value is the larger key, then the lower index; 0
    // (no expert left in the lane) loses to every candidate, and top <= E
    // leaves at least one, so bi is a valid expert index.
    uint64_t c = 0;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      const int e = q * 64 + lane;
      const uint64_t cq = (static_cast<uint64_t>(key[q]) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
      if (e < E && !((taken >> q) & 1u) && cq > c) c = cq;
    }
    c = wave_max_u64(c);
    const int bi = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(c));
    // its logit, from the lane and slot that hold it
    float vs = v[0];
#pragma unroll
    for (int q = 1; q < kMaxPer; ++q)
      if ((bi >> 6) == q) vs = v[q];
    const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vs), bi & 63));
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      ids[t * top + j] = bi;
      wts[t * top + j] = expf(bv - mx) / sum;
    }
  }
}

// E <= 256, one wave per token: every lane ranks its own logits against the
// token's E logits (held in LDS per wave).  rank(e) = number of logits that
// have a larger selection key (route_key), or an equal one at a lower expert
// index, so the ranks are a permutation of 0..E-1 and the experts of rank <
// top are the top-k in the order the repeated wave argmax gives.  The softmax statistics are those of k_route_topk, operation for
// operation.
template <int PER>
__global__ __launch_bounds__(256) void k_route_topk_rank(const float *logits, int64_t T, int E, int top,
                                                         int32_t *ids, float *wts) {
  __shared__ __attribute__((aligned(16))) uint32_t lv[4][64 * PER];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const bool valid = t < T;  // no early return: every wave reaches the barrier
  const float *row = logits + (valid ? t : 0) * E;
  float v[PER];
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = q * 64 + lane;
    v[q] = valid && e < E ? row[e] : -INFINITY;
    mx = fmaxf(mx, v[q]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (q * 64 + lane < E) sum += expf(v[q] - mx);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  uint32_t key[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    key[q] = route_key(v[q]);
    if (q * 64 + lane < E) lv[wave][q * 64 + lane] = key[q];
  }
  __syncthreads();
  uint32_t rank[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) rank[q] = 0;
  const uint32_t *lw = lv[wave];
  int j = 0;
  for (; j + 4 <= E; j += 4) {
    const uint4 o = *reinterpret_cast<const uint4 *>(lw + j);
    const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < PER; ++q)
        rank[q] += ov[u] > key[q] || (ov[u] == key[q] && j + u < q * 64 + lane);
  }
  for (; j < E; ++j) {
    const uint32_t o = lw[j];
#pragma unroll
    for (int q = 0; q < PER; ++q) rank[q] += o > key[q] || (o == key[q] && j < q * 64 + lane);
  }
  if (valid) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = q * 64 + lane;
      if (e < E && rank[q] < static_cast<uint32_t>(top)) {
        ids[t * top + rank[q]] = e;
        wts[t * top + rank[q]] = expf(v[q] - mx) / sum;
      }
    }
  }
}

__global__ __launch_bounds__(kTokBlk) void k_route_count(const int32_t *ids, int64_t T, int E, int top,
                                                         int32_t *blkcnt) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += kTokBlk) cnt[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokBlk + threadIdx.x;
  if (t < T)
    for (int j = 0; j < top; ++j) atomicAdd(&cnt[ids[t * top + j]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kTokBlk) blkcnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// Per expert e (thread e): the exclusive running count over token blocks,
// loaded eight blocks at a time so that the loads of a batch are in flight
// together; then an exclusive prefix over experts (wave scans and the wave
// totals) gives expert_offsets, which is added to every block's entry.
__global__ __launch_bounds__(1024) void k_route_scan(int32_t *blkcnt, int nblk, int E, int32_t *offsets) {
  __shared__ int32_t wtot[16];
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  constexpr int U = 8;
  int32_t run = 0;
  if (e < E) {
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = blkcnt[static_cast<int64_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        blkcnt[static_cast<int64_t>(b + u) * E + e] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      const int32_t c = blkcnt[static_cast<int64_t>(b) * E + e];
      blkcnt[static_cast<int64_t>(b) * E + e] = run;
      run += c;
    }
  }
  int32_t incl = run;  // 0 for threads past E
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wv; ++w) before += wtot[w];
  const int32_t excl = before + incl - run;
  if (e < E) offsets[e] = excl;
  if (e == E - 1) offsets[E] = excl + run;
  if (e < E) {
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = blkcnt[static_cast<int64_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) blkcnt[static_cast<int64_t>(b + u) * E + e] = c[u] + excl;
    }
    for (; b < nblk; ++b) blkcnt[static_cast<int64_t>(b) * E + e] += excl;
  }
}

__global__ __launch_bounds__(kTokBlk) void k_route_scatter(const int32_t *ids, int64_t T, int E, int top,
                                                           const int32_t *blkoff, int32_t *row_token,
                                                           int32_t *inverse) {
  extern __shared__ uint32_t bits[];  // [E][kTokBlk / 32]
  constexpr int W = kTokBlk / 32;
  for (int i = threadIdx.x; i < E * W; i += kTokBlk) bits[i] = 0;
  __syncthreads();
  const int tl = threadIdx.x;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokBlk + tl;
  if (t < T)
    for (int j = 0; j < top; ++j) atomicOr(&bits[ids[t * top + j] * W + (tl >> 5)], 1u << (tl & 31));
  __syncthreads();
  if (t >= T) return;
  for (int j = 0; j < top; ++j) {
    const int e = ids[t * top + j];
    int rank = 0;
    for (int w = 0; w < (tl >> 5); ++w) rank += __popc(bits[e * W + w]);
    rank += __popc(bits[e * W + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
    const int32_t pos = blkoff[static_cast<int64_t>(blockIdx.x) * E + e] + rank;
    row_token[pos] = static_cast<int32_t>(t);
    inverse[t * top + j] = pos;
  }
}

// T <= kTokBlk (one token block, e.g. decode): count, scan and scatter in
// one workgroup.  LDS: cnt[E] | bits[E][kTokBlk / 32] | pre[E].  Rows are
// ordered by (expert, token, slot) exactly as by the three kernels above: a
// token chooses an expert at most once, so a row's rank within its expert is
// the number of earlier tokens in the expert's bitmap.
__global__ __launch_bounds__(kTokBlk) void k_route_one_block(const int32_t *ids, int T, int E, int top,
                                                             int32_t *offsets, int32_t *row_token,
                                                             int32_t *inverse) {
  extern __shared__ int32_t lds_i[];
  constexpr int W = kTokBlk / 32;
  int32_t *cnt = lds_i;
  uint32_t *bits = reinterpret_cast<uint32_t *>(lds_i + E);
  int32_t *pre = lds_i + E + E * W;
  __shared__ int32_t wsum[kTokBlk / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // This token's experts, loaded together (top <= 16) while the tables clear.
  int32_t ex[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < top && t < T) ex[j] = ids[t * top + j];
  for (int i = t; i < E; i += kTokBlk) cnt[i] = 0;
  for (int i = t; i < E * W; i += kTokBlk) bits[i] = 0;
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < top) {
        atomicAdd(&cnt[ex[j]], 1);
        atomicOr(&bits[ex[j] * W + (t >> 5)], 1u << (t & 31));
      }
  }
  __syncthreads();
  // Exclusive prefix of cnt over experts: thread t owns experts [4t, 4t + 4).
  int32_t c[4], own = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    c[q] = e < E ? cnt[e] : 0;
    own += c[q];
  }
  const int32_t incl = static_cast<int32_t>(wave_scan<false>(static_cast<uint32_t>(own)));
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t run = incl - own;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e < E) {
      pre[e] = run;
      offsets[e] = run;
    }
    run += c[q];
  }
  if (t == kTokBlk - 1) offsets[E] = run;  // the last thread's running sum is the total
  __syncthreads();
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < top) {
      const int e = ex[j];
      int rank = 0;
      for (int w = 0; w < (t >> 5); ++w) rank += __popc(bits[e * W + w]);
      rank += __popc(bits[e * W + (t >> 5)] & ((1u << (t & 31)) - 1u));
      const int32_t pos = pre[e] + rank;
      row_token[pos] = t;
      inverse[t * top + j] = pos;
    }
  }
}

// The same sum for a compile-time top: every slot's index and weight, then
// every slot's row chunk, are loaded before the first multiply, so a thread
// has all its loads in flight at once; the sum keeps the slot order and the
// operations of k_combine, so the result is the same bit for bit.
template <int TOP, bool NT>
__global__ __launch_bounds__(256) void k_combine_top(const float *y, int64_t T, int64_t N, const int32_t *inverse,
                                                     const float *w, float *out) {
  const int64_t n4 = N / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= T * n4) return;
  const int64_t t = idx / n4, c = idx % n4;
  int32_t rows[TOP];
  float wj[TOP];
#pragma unroll
  for (int j = 0; j < TOP; ++j) {
    rows[j] = inverse[t * TOP + j];
    wj[j] = w[t * TOP + j];
  }
  float4 v[TOP];
#pragma unroll
  for (int j = 0; j < TOP; ++j) {
    typedef float f32x4_nt __attribute__((ext_vector_type(4)));
    const f32x4_nt *src = reinterpret_cast<const f32x4_nt *>(y + static_cast<int64_t>(rows[j]) * N) + c;
    const f32x4_nt t = NT ? __builtin_nontemporal_load(src) : *src;
    v[j] = make_float4(t[0], t[1], t[2], t[3]);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < TOP; ++j) {
    acc.x = acc.x + wj[j] * v[j].x;
    acc.y = acc.y + wj[j] * v[j].y;
    acc.z = acc.z + wj[j] * v[j].z;
    acc.w = acc.w + wj[j] * v[j].w;
  }
  reinterpret_cast<float4 *>(out + t * N)[c] = acc;
}

__global__ __launch_bounds__(256) void k_combine(const float *y, int64_t T, int top, int64_t N,
                                                 const int32_t *inverse, const float *w, float *out) {
  const int64_t n4 = N / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= T * n4) return;
  const int64_t t = idx / n4, c = idx % n4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < top; ++j) {
    const float wj = w[t * top + j];
    const float4 v = reinterpret_cast<const float4 *>(y + static_cast<int64_t>(inverse[t * top + j]) * N)[c];
    acc.x = acc.x + wj * v.x;
    acc.y = acc.y + wj * v.y;
    acc.z = acc.z + wj * v.z;
    acc.w = acc.w + wj * v.w;
  }
  reinterpret_cast<float4 *>(out + t * N)[c] = acc;
}

}  // namespace

size_t route_ws_bytes(int64_t T, int E) {
  const int64_t nblk = (T + kTokBlk - 1) / kTokBlk;
  return static_cast<size_t>(nblk) * E * sizeof(int32_t) + 256;
}

hipError_t launch_route(const float *logits, int64_t T, int E, int top, int32_t *ids, float *w,
                        int32_t *offsets, int32_t *row_token, int32_t *inverse, void *ws,
                        hipStream_t stream) {
  const int nblk = static_cast<int>((T + kTokBlk - 1) / kTokBlk);
  int32_t *blk = static_cast<int32_t *>(ws);
  if (T > 0) {
    // Ranking wins where there is throughput to gain (measured: 16384 tokens x
    // 64 experts 18 against 37 us); with few tokens and more than 64 experts
    // the argmax rounds are shorter (256 x 128: 11.8 against 13.3 us).
    const dim3 g((T + 3) / 4), b(256);
    const bool rank = E <= 64 || (E <= 256 && T >= 2048);
    if (rank && E <= 64) hipLaunchKernelGGL(k_route_topk_rank<1>, g, b, 0, stream, logits, T, E, top, ids, w);
    else if (rank && E <= 128) hipLaunchKernelGGL(k_route_topk_rank<2>, g, b, 0, stream, logits, T, E, top, ids, w);
    else if (rank) hipLaunchKernelGGL(k_route_topk_rank<4>, g, b, 0, stream, logits, T, E, top, ids, w);
    else if (E <= 128) hipLaunchKernelGGL(k_route_topk<2>, g, b, 0, stream, logits, T, E, top, ids, w);
    else if (E <= 256) hipLaunchKernelGGL(k_route_topk<4>, g, b, 0, stream, logits, T, E, top, ids, w);
    else if (E <= 512) hipLaunchKernelGGL(k_route_topk<8>, g, b, 0, stream, logits, T, E, top, ids, w);
    else hipLaunchKernelGGL(k_route_topk<16>, g, b, 0, stream, logits, T, E, top, ids, w);
    if (nblk > 1)
      hipLaunchKernelGGL(k_route_count, dim3(nblk), dim3(kTokBlk), E * sizeof(int32_t), stream, ids, T, E,
                         top, blk);
  }
  if (nblk == 1) {  // one token block: count, scan and scatter in one workgroup
    hipLaunchKernelGGL(k_route_one_block, dim3(1), dim3(kTokBlk),
                       static_cast<size_t>(E) * (2 + kTokBlk / 32) * sizeof(int32_t), stream, ids,
                       static_cast<int>(T), E, top, offsets, row_token, inverse);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, stream, blk, nblk, E, offsets);
  if (T > 0)
    hipLaunchKernelGGL(k_route_scatter, dim3(nblk), dim3(kTokBlk), E * (kTokBlk / 32) * sizeof(uint32_t),
                       stream, ids, T, E, top, blk, row_token, inverse);
  return hipGetLastError();
}

hipError_t launch_combine(const float *y, int64_t T, int top, int64_t N, const int32_t *inverse,
                          const float *w, float *out, hipStream_t stream) {
  const int64_t total = T * (N / 4);
  if (total > 0) {
    // y is read once: a large y (prefill: 1.07 GB) streams past the caches
    // with nontemporal loads (201 against 232 us); a small one (decode:
    // 16 MB, just written by the down GEMM) is read with plain loads.
    const bool stream_y = T * top * N * static_cast<int64_t>(sizeof(float)) > (int64_t(256) << 20);
    if (top == 8 && stream_y)
      hipLaunchKernelGGL((k_combine_top<8, true>), dim3((total + 255) / 256), dim3(256), 0, stream, y, T, N, inverse,
                         w, out);
    else if (top == 8)
      hipLaunchKernelGGL((k_combine_top<8, false>), dim3((total + 255) / 256), dim3(256), 0, stream, y, T, N, inverse,
                         w, out);
    else
      hipLaunchKernelGGL(k_combine, dim3((total + 255) / 256), dim3(256), 0, stream, y, T, top, N, inverse,
                         w, out);
  }
  return hipGetLastError();
}

}  // namespace quads
