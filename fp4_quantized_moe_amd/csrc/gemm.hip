// Token-permuted grouped expert GEMM for gfx950: NVFP4 W4A4 with the RAC
// segment (extended K), and the bf16-operand mode of the trainer's W4A16
// forward.
//
// QUADS technical summary, section 2.2-B: the residual correction of the
// selected channels is added to the quantized path while the native W4A4 GEMM
// keeps most of the work; the AI-Wiki "Methodology" section adds it before the
// GEMM.  Here that is one GEMM over an extended contraction:
//
//   Y[i,n] = gw[e,seg(n)] * ( gx * sum_k W[e,n,k] X[t(i),k]
//                           + gr * sum_j W[e,n,sel_j] R[t(i),j] )
//
// Operand decode.  An NVFP4 value e2m1 * e4m3 has at most 2 + 4 significant
// bits and lies in [2^-10, 2688], so it is exact in bf16; bf16 x bf16 products
// are exact in FP32, so a bf16 MFMA with FP32 accumulation computes the
// W4A4 sum with only accumulation rounding.  The block scales are 16-element
// E4M3, which the gfx950 scaled f8f6f4 MFMA (32-element power-of-two scales)
// cannot express exactly, so operands are decoded to bf16 on the way from
// global memory to LDS, once per workgroup tile:
//   - a 128-entry LDS table maps each E4M3 scale byte to the low and high
//     bytes of the bf16 values level_i * scale for the eight E2M1 levels;
//   - v_perm_b32 looks four 3-bit level indices up at once in that table, the
//     sign bits are OR-ed in, and two more v_perm_b32 interleave low/high
//     bytes into bf16 pairs: about 1.75 VALU operations per element.
//   The decode emits each 8-element group in the order 0,2,4,6,1,3,5,7.  A
//   contraction does not depend on the order of k, and both operands of a
//   W4A4 product use the same order; the gathered bf16 residual weights are
//   written in that order too.
//
// Tiling: 128x128 output tile, K step 64, 256 threads = 4 waves each owning a
// 64x64 sub-tile of 2x2 v_mfma_f32_32x32x16_bf16.  LDS holds double-buffered
// bf16 tiles [128][64] whose 16-byte chunks are XOR-swizzled by (row & 7) so
// that both the decode writes and the MFMA operand reads are conflict-free.
// Global loads for step k+1 are issued before the MFMAs of step k.
//
// Scheduling: a tile list over (expert, m-tile) is built on the device from
// expert_offsets (no host sync); the grid is an upper bound and surplus
// workgroups exit.  Workgroup ids are remapped so that each of the 8 XCDs
// (dispatched round-robin) owns a contiguous range of tiles, keeping an
// expert's weights and an m-tile's activations in one L2.
//
// RAC segment: the selected weight columns are gathered once per call into a
// bf16 [E, N, kpad] buffer (k_gather_wcols), after which the residual is a
// plain extended-K loop; the FP32 accumulator is rescaled by gx/gr between the
// two segments so a single accumulator serves both.
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Decode 8 E2M1 codes (one 32-bit word, element i in nibble i) with the
// per-scale table entry L = (lo bytes of levels 0-3, 4-7, hi bytes 0-3, 4-7)
// into 8 bf16 in the order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ uint4 decode8(uint32_t w, uint4 L) {
  const uint32_t sel_e = w & 0x07070707u;
  const uint32_t sel_o = (w >> 4) & 0x07070707u;
  const uint32_t lo_e = perm(L.y, L.x, sel_e);
  const uint32_t hi_e = perm(L.w, L.z, sel_e) | ((w << 4) & 0x80808080u);
  const uint32_t lo_o = perm(L.y, L.x, sel_o);
  const uint32_t hi_o = perm(L.w, L.z, sel_o) | (w & 0x80808080u);
  uint4 o;
  o.x = perm(hi_e, lo_e, 0x05010400u);
  o.y = perm(hi_e, lo_e, 0x07030602u);
  o.z = perm(hi_o, lo_o, 0x05010400u);
  o.w = perm(hi_o, lo_o, 0x07030602u);
  return o;
}

// Table entry for E4M3 scale byte s: bf16 of level_i * dec(s), split into
// low and high bytes.  Product of <= 2 and <= 4 significant bits: exact.
__device__ __forceinline__ uint4 make_lut_entry(uint32_t s) {
  uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
  if (s < 0x7Fu) {
    const float sc = e4m3_to_f32(s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = __float_as_uint(e2m1_level(i) * sc) >> 16;
      lo[i >> 2] |= (b & 0xFFu) << (8 * (i & 3));
      hi[i >> 2] |= (b >> 8) << (8 * (i & 3));
    }
  }
  return make_uint4(lo[0], lo[1], hi[0], hi[1]);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

struct Params {
  const int32_t *expert_offsets;
  const int32_t *tile_offsets;
  int E, n_seg, n_tiles, grid_per_xcd;
  int64_t N, K, kpad;
  const int32_t *row_token;
  const uint8_t *x_codes, *x_scales;
  const float *x_g;
  const uint8_t *r_codes, *r_scales;
  const float *r_g;
  const uint8_t *w_codes, *w_scales;
  const float *w_g;
  const uint16_t *x_bf16, *w_bf16, *wg_bf16;
  void *y;
  int y_bf16;
};

// ---- operand stagers -------------------------------------------------------
// NVFP4 rows: 128 rows x 4 blocks per K step; thread t stages blocks
// (row t/4 + 64p, block t%4), p = 0,1.
struct Fp4Stage {
  uint2 w[2];
  uint32_t s[2];
};

__device__ __forceinline__ void fp4_fetch(Fp4Stage &st, const uint8_t *codes, const uint8_t *scales,
                                          const int64_t (&row)[2], int64_t nblk, int kt) {
  const int64_t blk = static_cast<int64_t>(kt) * 4 + (threadIdx.x & 3);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (blk < nblk) {
      st.w[p] = *reinterpret_cast<const uint2 *>(codes + (row[p] * nblk + blk) * 8);
      st.s[p] = scales[row[p] * nblk + blk];
    } else {
      st.w[p] = make_uint2(0, 0);
      st.s[p] = 0;
    }
  }
}

__device__ __forceinline__ void fp4_store(const Fp4Stage &st, uint4 *tile, const uint4 *lut) {
  const int c = (threadIdx.x & 3) * 2;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = (threadIdx.x >> 2) + 64 * p;
    const uint4 L = lut[st.s[p] & 0x7Fu];
    tile[swz(r, c)] = decode8(st.w[p].x, L);
    tile[swz(r, c + 1)] = decode8(st.w[p].y, L);
  }
}

// bf16 rows: 128 rows x 8 chunks of 8 elements; thread t stages chunk t%8 of
// rows t/8 + 32q, q = 0..3.
struct Bf16Stage {
  uint4 v[4];
};

__device__ __forceinline__ void bf16_fetch(Bf16Stage &st, const uint16_t *base,
                                           const int64_t (&row)[4], int64_t ld, int64_t kdim,
                                           int kt) {
  const int64_t k = static_cast<int64_t>(kt) * BK + (threadIdx.x & 7) * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (k < kdim)
      st.v[q] = *reinterpret_cast<const uint4 *>(base + row[q] * ld + k);
    else
      st.v[q] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void bf16_store(const Bf16Stage &st, uint4 *tile) {
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int q = 0; q < 4; ++q) tile[swz((threadIdx.x >> 3) + 32 * q, c)] = st.v[q];
}

// One K step of MFMAs on the staged tiles.
__device__ __forceinline__ void mfma_step(const uint4 *As, const uint4 *Bs, f32x16 (&acc)[2][2],
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int chunk = 2 * ks + (lane >> 5);
    bf16x8 a[2], b[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      a[mi] = __builtin_bit_cast(bf16x8, As[swz(wm * 64 + mi * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      b[ni] = __builtin_bit_cast(bf16x8, Bs[swz(wn * 64 + ni * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
  }
}

// Weight row of tile row tr.  SWIGLU tiles interleave 32-row gate and up
// slices so each wave's 64 columns are 32 gate + the matching 32 up columns.
template <int EPI>
__device__ __forceinline__ int64_t w_row_of(int tr, int nt, int64_t N) {
  if constexpr (EPI == 0) {
    return static_cast<int64_t>(nt) * BN + tr;
  } else {
    const int64_t I = N / 2;
    return ((tr & 63) >> 5) * I + static_cast<int64_t>(nt) * 64 + (tr >> 6) * 32 + (tr & 31);
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// MODE 0: NVFP4 operands (+ residual segment if HAS_RES); MODE 1: bf16 operands.
template <int MODE, int EPI, bool HAS_RES>
__global__ __launch_bounds__(kThreads, 2) void k_gemm(Params p) {
  __shared__ uint4 As[2][BM * BK / 8];
  __shared__ uint4 Bs[2][BN * BK / 8];
  __shared__ uint4 lut[128];
  __shared__ int s_e, s_m0, s_mend;

  // XCD-aware remap: XCD x (= blockIdx % 8) gets logical tiles
  // [x * grid_per_xcd, (x + 1) * grid_per_xcd).
  const int logical = (blockIdx.x & 7) * p.grid_per_xcd + (blockIdx.x >> 3);
  const int mt = logical / p.n_tiles, nt = logical % p.n_tiles;
  if (mt >= p.tile_offsets[p.E]) return;
  if (threadIdx.x == 0) {
    int lo = 0, hi = p.E;  // largest e with tile_offsets[e] <= mt
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_offsets[mid] <= mt) lo = mid; else hi = mid;
    }
    s_e = lo;
    s_m0 = p.expert_offsets[lo] + (mt - p.tile_offsets[lo]) * BM;
    s_mend = p.expert_offsets[lo + 1];
  }
  if constexpr (MODE == 0) {
    for (int s = threadIdx.x; s < 128; s += kThreads) lut[s] = make_lut_entry(s);
  }
  __syncthreads();
  const int e = s_e, m0 = s_m0, mend = s_mend;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  auto act_row = [&](int r) -> int64_t {
    int i = m0 + r;
    if (i >= mend) i = mend - 1;  // padding rows re-read a valid row; never stored
    return p.row_token ? static_cast<int64_t>(p.row_token[i]) : static_cast<int64_t>(i);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int64_t wbase = static_cast<int64_t>(e) * p.N;  // expert's first weight row

  if constexpr (MODE == 0) {
    int64_t arow[2], brow[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      arow[q] = act_row((threadIdx.x >> 2) + 64 * q);
      brow[q] = wbase + w_row_of<EPI>((threadIdx.x >> 2) + 64 * q, nt, p.N);
    }
    const int64_t nblk = p.K / 16;
    const int nk = static_cast<int>((p.K + BK - 1) / BK);
    Fp4Stage sa, sb;
    fp4_fetch(sa, p.x_codes, p.x_scales, arow, nblk, 0);
    fp4_fetch(sb, p.w_codes, p.w_scales, brow, nblk, 0);
    fp4_store(sa, As[0], lut);
    fp4_store(sb, Bs[0], lut);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) {
        fp4_fetch(sa, p.x_codes, p.x_scales, arow, nblk, kt + 1);
        fp4_fetch(sb, p.w_codes, p.w_scales, brow, nblk, kt + 1);
      }
      mfma_step(As[cur], Bs[cur], acc, wm, wn, lane);
      if (kt + 1 < nk) {
        fp4_store(sa, As[cur ^ 1], lut);
        fp4_store(sb, Bs[cur ^ 1], lut);
      }
      __syncthreads();
    }
    if constexpr (HAS_RES) {
      const float ratio = *p.x_g / *p.r_g;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ratio;
      int64_t growb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) growb[q] = wbase + w_row_of<EPI>((threadIdx.x >> 3) + 32 * q, nt, p.N);
      const int64_t rblk = p.kpad / 16;
      const int nr = static_cast<int>((p.kpad + BK - 1) / BK);
      Fp4Stage sr;
      Bf16Stage sg;
      fp4_fetch(sr, p.r_codes, p.r_scales, arow, rblk, 0);
      bf16_fetch(sg, p.wg_bf16, growb, p.kpad, p.kpad, 0);
      fp4_store(sr, As[0], lut);
      bf16_store(sg, Bs[0]);
      __syncthreads();
      for (int kt = 0; kt < nr; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nr) {
          fp4_fetch(sr, p.r_codes, p.r_scales, arow, rblk, kt + 1);
          bf16_fetch(sg, p.wg_bf16, growb, p.kpad, p.kpad, kt + 1);
        }
        mfma_step(As[cur], Bs[cur], acc, wm, wn, lane);
        if (kt + 1 < nr) {
          fp4_store(sr, As[cur ^ 1], lut);
          bf16_store(sg, Bs[cur ^ 1]);
        }
        __syncthreads();
      }
    }
  } else {
    int64_t arow[4], brow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      arow[q] = act_row((threadIdx.x >> 3) + 32 * q);
      brow[q] = wbase + w_row_of<EPI>((threadIdx.x >> 3) + 32 * q, nt, p.N);
    }
    const int nk = static_cast<int>((p.K + BK - 1) / BK);
    Bf16Stage sa, sb;
    bf16_fetch(sa, p.x_bf16, arow, p.K, p.K, 0);
    bf16_fetch(sb, p.w_bf16, brow, p.K, p.K, 0);
    bf16_store(sa, As[0]);
    bf16_store(sb, Bs[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) {
        bf16_fetch(sa, p.x_bf16, arow, p.K, p.K, kt + 1);
        bf16_fetch(sb, p.w_bf16, brow, p.K, p.K, kt + 1);
      }
      mfma_step(As[cur], Bs[cur], acc, wm, wn, lane);
      if (kt + 1 < nk) {
        bf16_store(sa, As[cur ^ 1]);
        bf16_store(sb, Bs[cur ^ 1]);
      }
      __syncthreads();
    }
  }

  // ---- epilogue ----
  float ascale = 1.0f;
  if constexpr (MODE == 0) ascale = HAS_RES ? *p.r_g : *p.x_g;
  if constexpr (EPI == 0) {
    const int64_t seg_len = p.N / p.n_seg;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t col = static_cast<int64_t>(nt) * BN + wn * 64 + ni * 32 + (lane & 31);
      float sc = ascale;
      if constexpr (MODE == 0) sc = p.w_g[e * p.n_seg + col / seg_len] * ascale;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (i < mend) {
            const float v = acc[mi][ni][r] * sc;
            if (p.y_bf16)
              static_cast<uint16_t *>(p.y)[static_cast<int64_t>(i) * p.N + col] =
                  static_cast<uint16_t>(f32_to_bf16_bits(v));
            else
              static_cast<float *>(p.y)[static_cast<int64_t>(i) * p.N + col] = v;
          }
        }
    }
  } else {
    const int64_t I = p.N / 2;
    const int64_t col = static_cast<int64_t>(nt) * 64 + wn * 32 + (lane & 31);
    float sg = ascale, su = ascale;
    if constexpr (MODE == 0) {
      sg = p.w_g[e * 2] * ascale;
      su = p.w_g[e * 2 + 1] * ascale;
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (i < mend) {
          const float g = acc[mi][0][r] * sg;
          const float u = acc[mi][1][r] * su;
          static_cast<uint16_t *>(p.y)[static_cast<int64_t>(i) * I + col] =
              static_cast<uint16_t>(f32_to_bf16_bits(silu(g) * u));
        }
      }
  }
}

// Exclusive scan of per-expert m-tile counts -> tile_offsets[E + 1].
__global__ __launch_bounds__(1024) void k_tile_prefix(const int32_t *offsets, int E, int32_t *tile_offsets) {
  __shared__ int32_t sums[1025];
  const int t = threadIdx.x;
  int32_t v = 0;
  if (t < E) v = (offsets[t + 1] - offsets[t] + BM - 1) / BM;
  sums[t + 1] = v;
  if (t == 0) sums[0] = 0;
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i <= E; ++i) sums[i] += sums[i - 1];
  }
  __syncthreads();
  if (t < E) tile_offsets[t] = sums[t];
  if (t == 0) tile_offsets[E] = sums[E];
}

// Gather the selected weight columns of every expert row into bf16
// [E*N, kpad] (exact values e2m1 * e4m3, no tensor scale), each 8-element
// group in the decode order 0,2,4,6,1,3,5,7.  Two rows per workgroup.
__global__ __launch_bounds__(256) void k_gather_wcols(const uint8_t *w_codes, const uint8_t *w_scales,
                                                      int64_t rows_total, int K, const int32_t *sel,
                                                      int kpad, uint16_t *out) {
  extern __shared__ uint8_t lds[];
  const int half = threadIdx.x >> 7, t = threadIdx.x & 127;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 2 + half;
  const int rb = K / 2 + K / 16;
  uint8_t *mine = lds + half * ((rb + 15) / 16 * 16);
  if (row < rows_total) {
    const uint8_t *c = w_codes + row * (K / 2);
    for (int i = t; i < K / 8; i += 128)
      reinterpret_cast<uint32_t *>(mine)[i] = reinterpret_cast<const uint32_t *>(c)[i];
    const uint8_t *s = w_scales + row * (K / 16);
    for (int i = t; i < K / 16; i += 128) mine[K / 2 + i] = s[i];
  }
  __syncthreads();
  if (row >= rows_total) return;
  constexpr int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  for (int g = t; g < kpad / 8; g += 128) {
    uint32_t h[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = sel[g * 8 + order[q]];
      const uint32_t code = (mine[c >> 1] >> ((c & 1) * 4)) & 0xFu;
      const float v = e2m1_level(code & 7u) * e4m3_to_f32(mine[K / 2 + (c >> 4)]);
      h[q] = (__float_as_uint(v) >> 16) | ((code & 8u) << 12);
    }
    reinterpret_cast<uint4 *>(out + row * kpad)[g] =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  }
}

template <int MODE, int EPI, bool RES>
void launch_k(const Params &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm<MODE, EPI, RES>), dim3(grid), dim3(kThreads), 0, s, p);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t gemm_ws_bytes(const GemmLaunch &a) {
  size_t b = align256(static_cast<size_t>(a.E + 1) * sizeof(int32_t));
  if (a.mode == 0 && a.r_codes != nullptr && a.kpad > 0)
    b += align256(static_cast<size_t>(a.E) * a.N * a.kpad * sizeof(uint16_t));
  return b;
}

hipError_t launch_gemm(const GemmLaunch &a, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  int32_t *tile_offsets = reinterpret_cast<int32_t *>(ws);
  const bool res = a.mode == 0 && a.r_codes != nullptr && a.kpad > 0;
  uint16_t *wg = res ? reinterpret_cast<uint16_t *>(ws + align256((a.E + 1) * sizeof(int32_t))) : nullptr;
  hipLaunchKernelGGL(k_tile_prefix, dim3(1), dim3(1024), 0, stream, a.expert_offsets, a.E, tile_offsets);
  if (res) {
    const int64_t rows_total = static_cast<int64_t>(a.E) * a.N;
    const int K = static_cast<int>(a.K);
    const size_t lds = 2 * ((K / 2 + K / 16 + 15) / 16 * 16);
    hipLaunchKernelGGL(k_gather_wcols, dim3((rows_total + 1) / 2), dim3(256), lds, stream, a.w_codes,
                       a.w_scales, rows_total, K, a.sel_idx, static_cast<int>(a.kpad), wg);
  }
  Params p{};
  p.expert_offsets = a.expert_offsets;
  p.tile_offsets = tile_offsets;
  p.E = a.E;
  p.n_seg = a.n_seg;
  p.N = a.N;
  p.K = a.K;
  p.kpad = a.kpad;
  p.row_token = a.row_token;
  p.x_codes = a.x_codes;
  p.x_scales = a.x_scales;
  p.x_g = a.x_g;
  p.r_codes = a.r_codes;
  p.r_scales = a.r_scales;
  p.r_g = a.r_g;
  p.w_codes = a.w_codes;
  p.w_scales = a.w_scales;
  p.w_g = a.w_g;
  p.x_bf16 = a.x_bf16;
  p.w_bf16 = a.w_bf16;
  p.wg_bf16 = wg;
  p.y = a.y;
  p.y_bf16 = a.y_bf16 ? 1 : 0;
  p.n_tiles = static_cast<int>(a.epilogue == 0 ? a.N / BN : a.N / 128);
  const int64_t m_tiles = (a.num_rows + BM - 1) / BM + a.E;
  int64_t grid = m_tiles * p.n_tiles;
  grid = (grid + 7) / 8 * 8;
  p.grid_per_xcd = static_cast<int>(grid / 8);
  const int g = static_cast<int>(grid);
  if (a.mode == 1) {
    if (a.epilogue == 0) launch_k<1, 0, false>(p, g, stream);
    else launch_k<1, 1, false>(p, g, stream);
  } else if (res) {
    if (a.epilogue == 0) launch_k<0, 0, true>(p, g, stream);
    else launch_k<0, 1, true>(p, g, stream);
  } else {
    if (a.epilogue == 0) launch_k<0, 0, false>(p, g, stream);
    else launch_k<0, 1, false>(p, g, stream);
  }
  return hipGetLastError();
}

}  // namespace quads
