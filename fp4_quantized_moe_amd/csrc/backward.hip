// W4A16 QAT backward of the grouped expert linear on gfx950.
//
// QUADS technical summary, section 2.2-A: every trainer forward uses the
// NVFP4 fake-quantized weights W_qdq while the optimizer updates the bf16
// masters, so the gradient passes the QDQ unchanged (straight-through).
// For y[i] = W_qdq[e(i)] . x[t(i)] over routed rows i grouped by expert:
//
//   dxr[i] = dy[i] . W_qdq[e(i)]      a grouped GEMM over W_qdq^T: the
//                                     forward's bf16-operand GEMM once
//                                     k_transpose has written W_qdq^T;
//   dW[e]  = sum over the expert's rows i of dy[i]^T x[t(i)]   (k_wgrad).
//
// k_wgrad contracts over routed rows.  Those are strided in dy [R, N] and
// gathered in x [A, K].  So both operands are first written transposed
// with the routed rows along the contraction (k_pad_map + k_transpose in
// gather mode).  Each expert's rows are padded to a multiple of 64 with
// zeros, so every contraction step is whole and 16-byte aligned.  The
// weight-gradient kernel then has the forward's layout: rows of 16-byte
// chunks along the contraction, XOR-swizzled in LDS, on
// v_mfma_f32_32x32x16_bf16 with FP32 accumulation and an FP32 dW.
#include "fp4_mfma.hpp"
#include "launch.hpp"

namespace quads {
namespace {

constexpr int kPad = 64;   // per-expert row padding (a 64-column transpose tile stays in one expert)
constexpr int kStep = 64;  // contraction step of k_wgrad (divides kPad): one 128-byte line per row
constexpr int kCh = kStep / 8;  // 16-byte chunks per tile row and step

__device__ __forceinline__ int pad_up(int m) { return (m + kPad - 1) / kPad * kPad; }

// One workgroup per expert e: pad_off[e] = sum over e' < e of pad_up(rows of
// e'), colsrc[pad_off[e] + j] = the expert's j-th routed row (or -1 in the
// padding) and colexp[pad_off[e] + j] = e.  The last workgroup also writes
// pad_off[E].
__global__ __launch_bounds__(256) void k_pad_map(const int32_t *offsets, int E, int32_t *pad_off,
                                                 int32_t *colsrc, int32_t *colexp) {
  __shared__ int32_t wsum[4];
  const int e = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t own = 0;
  for (int i = t; i < e; i += 256) own += pad_up(offsets[i + 1] - offsets[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) own += __shfl_xor(own, off);
  if (lane == 0) wsum[wave] = own;
  __syncthreads();
  const int32_t p = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int32_t a = offsets[e], m = offsets[e + 1] - a, mp = pad_up(m);
  for (int j = t; j < mp; j += 256) {
    colsrc[p + j] = j < m ? a + j : -1;
    colexp[p + j] = e;
  }
  if (t == 0) {
    pad_off[e] = p;
    if (e == E - 1) pad_off[E] = p + mp;
  }
}

// out[b][c][j] = in[b][src(j)][c] for a 64 x 64 tile of (c, j), bf16.
// src(j) = j (plain transpose), or in gather mode colsrc[j] mapped through
// row_token (when given), with -1 giving a zero column.  Columns j >= pad_off[E]
// (gather mode: the padded row count known only on the device) are not
// written.  rows (J) and cols (C) are multiples of 8: every 16-byte chunk is
// whole.  The LDS tile has 66-element rows: the column reads of the second
// phase then hit distinct banks (33 words per row).
// Gather mode writes one contiguous block per expert: expert e's padded
// columns [pad_off[e], pad_off[e+1]) go to out + C * pad_off[e] as a
// [C, pad_off[e+1] - pad_off[e]] matrix.  A 64-column tile lies inside one
// expert because every expert's range is 64-aligned.
template <bool GATHER>
__global__ __launch_bounds__(256) void k_transpose(const uint16_t *in, int64_t C, int64_t J, int64_t in_bstride,
                                                   const int32_t *colsrc, const int32_t *row_token,
                                                   const int32_t *pad_off, const int32_t *colexp, int E,
                                                   uint16_t *out, int64_t ld_out, int64_t out_bstride) {
  __shared__ uint16_t tile[64][66];
  const int t = threadIdx.x;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int64_t Jn = GATHER ? min(J, static_cast<int64_t>(pad_off[E])) : J;
  if (j0 >= Jn) return;
  const uint16_t *src = in + static_cast<int64_t>(blockIdx.z) * in_bstride;
  uint16_t *dst = out + static_cast<int64_t>(blockIdx.z) * out_bstride;
  int64_t jbase = 0;  // first column of the output block this tile writes into
  if constexpr (GATHER) {
    const int e = colexp[j0];
    jbase = pad_off[e];
    ld_out = pad_off[e + 1] - jbase;
    dst += C * jbase;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int jj = t / 8 + 32 * q, ch = t % 8;
    const int64_t j = j0 + jj, c = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < Jn && c < C) {
      int64_t r = j;
      if constexpr (GATHER) {
        const int32_t i = colsrc[j];
        r = i < 0 ? -1 : (row_token ? row_token[i] : i);
      }
      if (r >= 0) v = *reinterpret_cast<const uint4 *>(src + r * C + c);
    }
    uint32_t *w = reinterpret_cast<uint32_t *>(&tile[jj][ch * 8]);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int cc = t / 8 + 32 * q, jc = t % 8;
    const int64_t c = c0 + cc, j = j0 + jc * 8;
    if (c >= C || j >= Jn) continue;
    uint32_t h[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      h[m] = static_cast<uint32_t>(tile[jc * 8 + 2 * m][cc]) | (static_cast<uint32_t>(tile[jc * 8 + 2 * m + 1][cc]) << 16);
    *reinterpret_cast<uint4 *>(dst + c * ld_out + (j - jbase)) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

// dW[e, n, k] = sum over j in [pad_off[e], pad_off[e+1]) of dyT[n, j] * xT[k, j].
// Workgroup tile TN (n) x TK (k) of WN x WK waves (256 x 256 with 8 waves of
// 128 x 64 where N and K allow, else 128 x 128 with 4 waves of 64 x 64): the
// larger tile halves the operand re-reads, which (an expert's two transposed
// blocks being larger than one XCD's L2) set this kernel's speed.
// Contraction steps of 64: each staging load instruction reads whole
// 128-byte lines (8 lanes per row; a load spread over 64 bytes of each of
// 16 rows streams at about half that rate on MI355X).  LDS rows hold 8
// chunks, chunk c of row r in slot c ^ ((r >> 1) & 7), which keeps the 16
// rows a fragment read touches at one chunk, and the 2 rows x 8 chunks a store
// instruction's 16 lanes write, in distinct 16-byte bank groups.  Two LDS stages; the next step's loads
// are in flight while a step is multiplied.  The workgroup order keeps all
// tiles of an expert on one XCD (dispatch is round-robin over the 8 XCDs).
// Each expert's operand blocks are contiguous ([N, padded rows] and
// [K, padded rows]), so a tile's rows lie in one region of memory.
template <int TN, int TK>
struct WgradLds {
  uint4 a[TN * kCh];
  uint4 b[TK * kCh];
};

__device__ __forceinline__ int wslot(int row, int c) { return row * kCh + (c ^ ((row / (16 / kCh)) & (kCh - 1))); }

template <int TN, int TK, int WN, int WK>
struct WgradCfg {
  static constexpr int THREADS = 64 * WN * WK;
  static constexpr int LA = TN * kCh / THREADS, LB = TK * kCh / THREADS;  // staging loads per thread
  static constexpr int RS = THREADS / kCh;                               // tile rows between them
  static constexpr int MI = TN / WN / 32, KI = TK / WK / 32;              // 32x32 MFMA tiles per wave
  static_assert(LA >= 1 && LB >= 1 && TN * kCh % THREADS == 0 && TK * kCh % THREADS == 0, "staging split");
};

template <class C, int TN, int TK>
__device__ __forceinline__ void wg_fetch(uint4 (&ra)[C::LA], uint4 (&rb)[C::LB], const uint16_t *ga,
                                         const uint16_t *gb, int64_t ld, int s) {
  const int64_t o = static_cast<int64_t>(s) * kStep;
#pragma unroll
  for (int q = 0; q < C::LA; ++q) ra[q] = *reinterpret_cast<const uint4 *>(ga + C::RS * q * ld + o);
#pragma unroll
  for (int q = 0; q < C::LB; ++q) rb[q] = *reinterpret_cast<const uint4 *>(gb + C::RS * q * ld + o);
}

template <class C, int TN, int TK>
__device__ __forceinline__ void wg_store(WgradLds<TN, TK> &l, const uint4 (&ra)[C::LA], const uint4 (&rb)[C::LB],
                                         int srow, int sch) {
#pragma unroll
  for (int q = 0; q < C::LA; ++q) l.a[wslot(srow + C::RS * q, sch)] = ra[q];
#pragma unroll
  for (int q = 0; q < C::LB; ++q) l.b[wslot(srow + C::RS * q, sch)] = rb[q];
}

// One contraction step of this wave's (32 MI) x (32 KI) sub-tile.
template <class C, int TN, int TK>
__device__ __forceinline__ void wg_compute(const WgradLds<TN, TK> &l, f32x16 (&acc)[C::MI][C::KI], int an0,
                                           int bk0, int fr, int fh) {
#pragma unroll
  for (int sub = 0; sub < kCh / 2; ++sub) {
    const int c = 2 * sub + fh;
    uint4 a[C::MI], b[C::KI];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) a[i] = l.a[wslot(an0 + i * 32 + fr, c)];
#pragma unroll
    for (int i = 0; i < C::KI; ++i) b[i] = l.b[wslot(bk0 + i * 32 + fr, c)];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int ki = 0; ki < C::KI; ++ki)
        acc[mi][ki] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[mi]),
                                                              __builtin_bit_cast(bf16x8, b[ki]), acc[mi][ki], 0, 0, 0);
  }
}

template <int TN, int TK, int WN, int WK>
__global__ __launch_bounds__(64 * WN * WK) void k_wgrad(const uint16_t *dyT, const uint16_t *xT,
                                                        const int32_t *pad_off, int64_t N, int64_t K, float *dw) {
  using C = WgradCfg<TN, TK, WN, WK>;
  __shared__ WgradLds<TN, TK> st[2];
  const int nN = static_cast<int>(N / TN), nK = static_cast<int>(K / TK);
  const int G = gridDim.x;
  const int bid = G % 8 == 0 ? static_cast<int>((blockIdx.x % 8) * (G / 8) + blockIdx.x / 8)
                             : static_cast<int>(blockIdx.x);
  const int e = bid / (nN * nK), nb = (bid / nK) % nN, kb = bid % nK;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wn = wave / WK, wk = wave % WK;
  const int64_t n0 = static_cast<int64_t>(nb) * TN, k0 = static_cast<int64_t>(kb) * TK;
  const int j_begin = pad_off[e], j_end = pad_off[e + 1];
  const int64_t ld = j_end - j_begin;  // the expert's block: [N, ld] of dyT, [K, ld] of xT
  const int ns = static_cast<int>(ld / kStep);

  // Thread t stages chunk t % kCh of rows t / kCh + RS * q of both operands.
  const int srow = t / kCh, sch = t % kCh;
  const uint16_t *ga = dyT + N * j_begin + (n0 + srow) * ld + sch * 8;
  const uint16_t *gb = xT + K * j_begin + (k0 + srow) * ld + sch * 8;
  const int fr = lane & 31, fh = lane >> 5;
  const int an0 = wn * (TN / WN), bk0 = wk * (TK / WK);

  f32x16 acc[C::MI][C::KI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ki = 0; ki < C::KI; ++ki)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ki][r] = 0.0f;

  // Step s+1 loads into registers while step s is multiplied from its LDS
  // stage; the registers then go to the other stage.  The last step's
  // prefetch re-reads that step (in bounds) into a stage no one reads again,
  // so the loop body has no branches (with a branch the compiler kept the
  // staging registers in scratch memory).
  if (ns > 0) {
    uint4 ra[C::LA], rb[C::LB];
    wg_fetch<C, TN, TK>(ra, rb, ga, gb, ld, 0);
    wg_store<C, TN, TK>(st[0], ra, rb, srow, sch);
    __syncthreads();
    for (int s = 0; s < ns; ++s) {
      wg_fetch<C, TN, TK>(ra, rb, ga, gb, ld, min(s + 1, ns - 1));
      wg_compute<C, TN, TK>(st[s & 1], acc, an0, bk0, fr, fh);
      wg_store<C, TN, TK>(st[(s + 1) & 1], ra, rb, srow, sch);
      __syncthreads();
    }
  }

  // Element r of a 32x32 accumulator: row 8*(r/4) + 4*(lane/32) + r%4 (n),
  // column lane%32 (k).
  float *out = dw + static_cast<int64_t>(e) * N * K;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ki = 0; ki < C::KI; ++ki)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t n = n0 + an0 + mi * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
        const int64_t k = k0 + bk0 + ki * 32 + fr;
        out[n * K + k] = acc[mi][ki][r];
      }
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

int64_t wgrad_padded_cols(int64_t R, int E) { return round_up(R + static_cast<int64_t>(kPad - 1) * E, 64); }

size_t wgrad_ws_bytes(int64_t R, int E, int64_t N, int64_t K) {
  const int64_t J = wgrad_padded_cols(R, E);
  return static_cast<size_t>(round_up(4 * (E + 1), 256) + 2 * round_up(4 * J, 256) + 2 * (N + K) * J);
}

hipError_t launch_transpose_bf16(const uint16_t *in, int64_t batch, int64_t rows, int64_t cols, uint16_t *out,
                                 hipStream_t stream) {
  if (batch == 0 || rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + 63) / 64), static_cast<unsigned>((cols + 63) / 64),
                  static_cast<unsigned>(batch));
  hipLaunchKernelGGL((k_transpose<false>), grid, dim3(256), 0, stream, in, cols, rows, rows * cols, nullptr,
                     nullptr, nullptr, nullptr, 0, out, rows, rows * cols);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradLaunch &a, hipStream_t stream) {
  const int64_t J = wgrad_padded_cols(a.R, a.E);
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  int32_t *pad_off = reinterpret_cast<int32_t *>(ws);
  int32_t *colsrc = reinterpret_cast<int32_t *>(ws + round_up(4 * (a.E + 1), 256));
  int32_t *colexp = reinterpret_cast<int32_t *>(ws + round_up(4 * (a.E + 1), 256) + round_up(4 * J, 256));
  uint16_t *dyT = reinterpret_cast<uint16_t *>(ws + round_up(4 * (a.E + 1), 256) + 2 * round_up(4 * J, 256));
  uint16_t *xT = dyT + a.N * J;
  hipLaunchKernelGGL(k_pad_map, dim3(a.E), dim3(256), 0, stream, a.expert_offsets, a.E, pad_off, colsrc, colexp);
  const unsigned jt = static_cast<unsigned>(J / 64);
  hipLaunchKernelGGL((k_transpose<true>), dim3(jt, static_cast<unsigned>((a.N + 63) / 64), 1), dim3(256), 0,
                     stream, a.dy, a.N, J, int64_t(0), colsrc, nullptr, pad_off, colexp, a.E, dyT, int64_t(0),
                     int64_t(0));
  hipLaunchKernelGGL((k_transpose<true>), dim3(jt, static_cast<unsigned>((a.K + 63) / 64), 1), dim3(256), 0,
                     stream, a.x, a.K, J, int64_t(0), colsrc, a.row_token, pad_off, colexp, a.E, xT, int64_t(0),
                     int64_t(0));
  if (a.N % 256 == 0 && a.K % 256 == 0) {
    const int64_t grid = static_cast<int64_t>(a.E) * (a.N / 256) * (a.K / 256);
    hipLaunchKernelGGL((k_wgrad<256, 256, 2, 4>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream, dyT, xT,
                       pad_off, a.N, a.K, a.dw);
  } else {
    const int64_t grid = static_cast<int64_t>(a.E) * (a.N / 128) * (a.K / 128);
    hipLaunchKernelGGL((k_wgrad<128, 128, 2, 2>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, dyT, xT,
                       pad_off, a.N, a.K, a.dw);
  }
  return hipGetLastError();
}

}  // namespace quads
