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
// bits and lies in [2^-10, 2688]: it is exact in fp16 (normal range
// [2^-14, 65504]), and fp16 x fp16 products are exact in FP32, so an fp16 MFMA
// with FP32 accumulation computes the W4A4 sum with only accumulation
// rounding.  The block scales are 16-element E4M3, which the gfx950 scaled
// f8f6f4 MFMA (32-element power-of-two scales) cannot express exactly, so
// operands are decoded on the way from global memory to LDS, once per
// workgroup tile: v_cvt_scalef32_pk_f16_fp4 (unit scale) turns two codes into
// two fp16 levels, and one v_pk_mul_f16 by the block scale (v_cvt of the E4M3
// byte, exact) gives the exact products -- two VALU operations per two
// elements.  The bf16-operand (trainer) mode feeds bf16 MFMAs directly.
//
// Tiling: templated BM x BN workgroup tiles of WGM x WGN waves, K step 64,
// v_mfma_f32_32x32x16_{f16,bf16}.  LDS holds two [rows][64] tiles per operand
// whose 16-byte chunks are XOR-swizzled by ((row >> 1) & 7) so that both the
// decode writes and the MFMA operand reads are conflict-free.  Global data is
// fetched two K steps ahead into alternating register stages; the loop body
// (fetch step k+2, MFMAs on step k, decode+store step k+1, barrier) has no
// branches, so the next step's decode can be interleaved with this step's
// MFMAs.
//
// Scheduling: a per-expert tile list is built on the device from
// expert_offsets (no host sync); the grid is an upper bound and surplus
// workgroups exit.  Workgroup ids are remapped so that each of the 8 XCDs
// (dispatched round-robin) owns a contiguous range of tiles, keeping an
// expert's weights and an m-tile's activations in one L2.
//
// RAC segment: the selected weight columns are gathered once per call into an
// fp16 [E, N, kpad] buffer (k_gather_wcols), after which the residual is a
// plain extended-K loop; the FP32 accumulator is rescaled by gx/gr between the
// two segments so a single accumulator serves both.
#include <stdlib.h>
#include <string.h>

#include "dma.hpp"
#include "fp4_mfma.hpp"
#include "launch.hpp"
#include "quads_device.hpp"

namespace quads {
namespace {

constexpr int BK = 64;  // K step: 4 NVFP4 blocks = 8 chunks of 8 16-bit values per row

// Workgroup tile BM x BN, WGM x WGN waves, each wave owning a (BM/WGM) x
// (BN/WGN) sub-tile of 32x32 MFMA tiles.
template <int BM_, int BN_, int WGM_, int WGN_, int MINB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int MINB = MINB_;  // workgroups per CU the register budget must allow
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int TM = BM / WGM, TN = BN / WGN;
  static constexpr int MI = TM / 32, NI = TN / 32;
  static constexpr int FA = BM * 4 / THREADS, FB = BN * 4 / THREADS;  // NVFP4 block loads / thread
  static constexpr int HA = BM * 8 / THREADS, HB = BN * 8 / THREADS;  // 16-byte raw loads / thread
  static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "wave tile must be 32-aligned");
  static_assert(FA * THREADS == BM * 4 && FB * THREADS == BN * 4, "fp4 staging must divide");
  static_assert(HA * THREADS == BM * 8 && HB * THREADS == BN * 8, "raw staging must divide");
};

// LDS tiles are [rows][8 chunks of 16 bytes]; chunk c of row r lives at
// c ^ ((r >> 1) & 7).  gfx950's LDS has 64 four-byte banks, so one bank row
// spans two 128-byte tile rows and 16 lanes of a 16-byte access are serviced
// together: with this swizzle the 16 consecutive rows read at one logical
// chunk (MFMA fragments) and the 2-4 rows x 4-8 chunks written by a
// decode/store instruction all land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

struct Params {
  const int32_t *expert_offsets;
  const int32_t *tile_offsets;  // per-expert prefix of BM-row m-tiles
  int E, n_seg, n_tiles;
  int64_t N, K, kpad;
  int64_t act_rows;  // rows of the activation tensors
  const int32_t *row_token;
  const uint8_t *x_codes, *x_scales;
  const float *x_g;
  const uint8_t *r_codes, *r_scales;
  const float *r_g;
  const uint8_t *w_codes, *w_scales;
  const float *w_g;
  const uint16_t *x_bf16, *w_bf16, *wg_f16;
  const uint16_t *x_f16;  // MODE 2: RAC-merged fp16 activation [act_rows, K], units of x_g
  void *y;
  int y_bf16;
  uint32_t *amax_ws;  // zeroed words gathering the amax of bf16 y when its tensor scale is wanted, else null
};

// MODE 3 weight rows: bf16 master values, fake-quantized (QDQ) to NVFP4 and
// back to bf16 on the way into LDS, with the tensor scale of their (expert,
// segment).  A 16-element block of a row is two 8-value chunks held by the
// lane pair (2j, 2j+1) -- chunk c of a row is staged by the lane with
// threadIdx & 7 == c -- so each lane takes its half's max and the pair
// exchanges it (DPP quad permute [1,0,3,2]).  Every lane runs the exchange,
// so no lane sits out of the DPP.
__device__ __forceinline__ uint4 qdq_chunk(const uint4 &v, bool ok, const TensorScale &g) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false));
  m = fmaxf(m, other);
  const uint4 q = qdq8_bf16(x, m, g);
  return ok ? q : make_uint4(0, 0, 0, 0);
}

// MODE 4 weight rows: NVFP4 codes and block scales decoded to their QDQ bf16
// values bf16(fl32(level * fl32(dec(s) * g))) -- the values quads_weight_qdq
// writes for the same codes -- as two 8-value chunks of one 16-block.  A
// block past the end of K stores zeros.
__device__ __forceinline__ void qdq_decode16(const uint2 &w, uint32_t s, float g, bool ok, uint4 &c0, uint4 &c1) {
  const float d = e4m3_to_f32(s) * g;
  float dq[8];
  dequant8(w.x, d, dq);
  c0 = ok ? make_uint4(pack_bf16x2(dq[0], dq[1]), pack_bf16x2(dq[2], dq[3]), pack_bf16x2(dq[4], dq[5]),
                       pack_bf16x2(dq[6], dq[7]))
          : make_uint4(0, 0, 0, 0);
  dequant8(w.y, d, dq);
  c1 = ok ? make_uint4(pack_bf16x2(dq[0], dq[1]), pack_bf16x2(dq[2], dq[3]), pack_bf16x2(dq[4], dq[5]),
                       pack_bf16x2(dq[6], dq[7]))
          : make_uint4(0, 0, 0, 0);
}

// Tensor scale of weight row `wrow` of expert e (segment = wrow / (N/n_seg)).
__device__ __forceinline__ float w_scale_of(const Params &p, int e, int64_t wrow) {
  return p.w_g[e * p.n_seg + wrow / (p.N / p.n_seg)];
}

// ---- operand stagers -------------------------------------------------------
// NVFP4 rows: 4 blocks per row per K step; thread t stages blocks
// (row fp4_row(t) + p*THREADS/4, block t%4).  `base[p]` is the row's first block
// index.  Loads are unconditional: a block past the end of K re-reads block 0
// of its row (in bounds) and is zeroed when decoded, so no branch or early
// wait sits between a fetch and its use two steps later.
template <int P>
struct Fp4Stage {
  uint2 w[P];
  uint32_t s[P];
  bool ok;
};

template <int P>
__device__ __forceinline__ void fp4_fetch(Fp4Stage<P> &st, const uint8_t *codes, const uint8_t *scales,
                                          const int64_t (&base)[P], int nblk, int kt, int part = -1) {
  const int blk = kt * 4 + (threadIdx.x & 3);
  st.ok = blk < nblk;
  const int off = st.ok ? blk : 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (part >= 0 && p % 4 != part) continue;
    st.w[p] = *reinterpret_cast<const uint2 *>(codes + (base[p] + off) * 8);
    st.s[p] = scales[base[p] + off];
  }
}

// Decode and store the blocks p of the stage with p % 4 == part (the store is
// split in four parts so each can follow one MFMA sub-step; the fetches take
// the same parts, part -1 being the whole stage).
// Row staged by thread t's lane quad: bits 0 and 1 of the quad index t/4 are
// swapped, so each group of 8 lanes (the granularity at which a 16-byte LDS
// write is serviced) covers two rows whose swizzle keys differ in bit 0 and
// the chunk sets {0,2,4,6} and {1,3,5,7} it writes do not collide.
__device__ __forceinline__ int fp4_row(int t) {
  const int q = t >> 2;
  return (q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1);
}

template <int P, int THREADS>
__device__ __forceinline__ void fp4_store(const Fp4Stage<P> &st, uint4 *tile, int part) {
  const int c = (threadIdx.x & 3) * 2;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p % 4 != part) continue;
    const int r = fp4_row(threadIdx.x) + p * (THREADS / 4);
    const h2 sc = scale_h2(st.ok ? st.s[p] : 0u);
    tile[swz(r, c)] = decode8_f16(st.w[p].x, sc);
    tile[swz(r, c + 1)] = decode8_f16(st.w[p].y, sc);
  }
}

// 16-bit rows (bf16 or pre-decoded fp16): 8 chunks of 8 values per row per K
// step; thread t stages chunk t%8 of rows t/8 + q*THREADS/8.  `base[q]` is the
// row's first element; same unconditional-load rule as above.
template <int P>
struct RawStage {
  uint4 v[P];
  bool ok;
};

template <int P>
__device__ __forceinline__ void raw_fetch(RawStage<P> &st, const uint16_t *src, const int64_t (&base)[P],
                                          int kdim, int kt, int part = -1) {
  const int k = kt * BK + (threadIdx.x & 7) * 8;
  st.ok = k < kdim;
  const int off = st.ok ? k : 0;
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (part < 0 || q % 4 == part) st.v[q] = *reinterpret_cast<const uint4 *>(src + base[q] + off);
}

// ZERO: chunks past the end of K are stored as zeros.  An activation operand
// whose weight operand is zeroed there (every NVFP4 or bf16 weight stager
// here) skips it: its re-read in-bounds values meet zero weights.
// Buffer-resource forms of the two fetchers (large tiles): each lane's byte
// offset inside the resource is fixed for the tile and the K step goes into
// the scalar offset, so a step's loads take no address arithmetic.  Reads
// past the resource's end return 0, and the stagers zero what lies past K,
// so no offset is clamped.  Offsets and sizes fit 32 bits (host-checked).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int64_t bytes) {
  // word 3: 32-bit data format (gfx9 raw buffer)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}

// blk0[p]: the lane's first block index in the resource (row * nblk + t % 4).
template <int P>
__device__ __forceinline__ void fp4_fetch_buf(Fp4Stage<P> &st, __amdgpu_buffer_rsrc_t codes,
                                              __amdgpu_buffer_rsrc_t scales, const uint32_t (&blk0)[P], int nblk,
                                              int kt, int part) {
  st.ok = kt * 4 + (threadIdx.x & 3) < nblk;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (part >= 0 && p % 4 != part) continue;
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(codes, blk0[p] * 8u, kt * 32, 0);
    st.w[p] = make_uint2(w[0], w[1]);
    st.s[p] = __builtin_amdgcn_raw_buffer_load_b8(scales, blk0[p], kt * 4, 0);
  }
}

// ofs[q]: the lane's byte offset of step 0 (2 * (row * kdim + (t % 8) * 8)).
template <int P>
__device__ __forceinline__ void raw_fetch_buf(RawStage<P> &st, __amdgpu_buffer_rsrc_t src, const uint32_t (&ofs)[P],
                                              int kdim, int kt, int part) {
  st.ok = kt * BK + (threadIdx.x & 7) * 8 < kdim;
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (part < 0 || q % 4 == part) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(src, ofs[q], kt * (2 * BK), 0);
      st.v[q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

template <int P, int THREADS, bool ZERO = true>
__device__ __forceinline__ void raw_store(const RawStage<P> &st, uint4 *tile, int part) {
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (q % 4 == part)
      tile[swz((threadIdx.x >> 3) + q * (THREADS / 8), c)] = (!ZERO || st.ok) ? st.v[q] : make_uint4(0, 0, 0, 0);
}

template <int P, int THREADS>
__device__ __forceinline__ void fp4_qdq_store(const Fp4Stage<P> &st, uint4 *tile, int part, const float (&g)[P]) {
  const int c = (threadIdx.x & 3) * 2;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p % 4 != part) continue;
    const int r = fp4_row(threadIdx.x) + p * (THREADS / 4);
    uint4 c0, c1;
    qdq_decode16(st.w[p], st.s[p], g[p], st.ok, c0, c1);
    tile[swz(r, c)] = c0;
    tile[swz(r, c + 1)] = c1;
  }
}

template <int P, int THREADS>
__device__ __forceinline__ void qdq_store(const RawStage<P> &st, uint4 *tile, int part, const TensorScale (&g)[P]) {
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (q % 4 == part) tile[swz((threadIdx.x >> 3) + q * (THREADS / 8), c)] = qdq_chunk(st.v[q], st.ok, g[q]);
}

// Operand fragments of one 16-wide K sub-step for this wave.
template <class C>
struct Frags {
  uint4 a[C::MI], b[C::NI];
};

template <class C>
__device__ __forceinline__ void load_frags(Frags<C> &f, const uint4 *As, const uint4 *Bs, int ks, int wm, int wn,
                                           int lane) {
  const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) f.a[mi] = As[swz(wm * C::TM + mi * 32 + (lane & 31), chunk)];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) f.b[ni] = Bs[swz(wn * C::TN + ni * 32 + (lane & 31), chunk)];
}

// The weight fragment is the MFMA's first operand and the activation the
// second, so each accumulator holds a 32x32 block of Y transposed: lane l has
// output row l % 32 and, in registers 4j..4j+3, the four consecutive columns
// 8j + 4(l / 32) + 0..3, which the epilogue stores as one vector.
template <class C, bool F16>
__device__ __forceinline__ void mfmas(const Frags<C> &f, f32x16 (&acc)[C::MI][C::NI]) {
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      if constexpr (F16)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, f.b[ni]),
                                                             __builtin_bit_cast(h8, f.a[mi]), acc[mi][ni], 0, 0, 0);
      else
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, f.b[ni]), __builtin_bit_cast(bf16x8, f.a[mi]), acc[mi][ni], 0, 0, 0);
    }
}

// One K step: four 16-wide sub-steps.  The fragments of sub-step ks+1 are
// read from LDS before the MFMAs of sub-step ks are issued, and part ks of the
// next step's decode/store follows them, so LDS latency and the decode VALU
// overlap the MFMAs; scheduling fences keep the compiler from regrouping the
// sub-steps (which would hoist every load and exhaust the register file).
template <class C, bool F16, class Store>
__device__ __forceinline__ void mfma_step(const uint4 *As, const uint4 *Bs, f32x16 (&acc)[C::MI][C::NI], int wm,
                                          int wn, int lane, Store store_part) {
  Frags<C> f0, f1;
  load_frags<C>(f0, As, Bs, 0, wm, wn, lane);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    Frags<C> &cur = (ks & 1) ? f1 : f0;
    Frags<C> &nxt = (ks & 1) ? f0 : f1;
    if (ks + 1 < BK / 16) load_frags<C>(nxt, As, Bs, ks + 1, wm, wn, lane);
    mfmas<C, F16>(cur, acc);
    store_part(ks);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Weight row of tile row tr.  For SWIGLU each wave's TN columns are TN/2
// gate columns followed by the matching TN/2 up columns, so both halves of
// an output element land in the same lane and register.
template <class C, int EPI>
__device__ __forceinline__ int64_t w_row_of(int tr, int nt, int64_t N) {
  if constexpr (EPI == 0) {
    return static_cast<int64_t>(nt) * C::BN + tr;
  } else {
    constexpr int half = C::TN / 2;
    const int wn = tr / C::TN, c = tr % C::TN;
    const int64_t hc = static_cast<int64_t>(nt) * (C::BN / 2) + wn * half + (c % half);
    return (c / half) * (N / 2) + hc;
  }
}


// Branch-free two-buffer pipeline.  Before half h of an iteration, LDS buffer
// h holds step kt+h and register stage 1-h holds step kt+h+1 (fetched one
// step earlier); half h runs the MFMAs on buffer h and, after each of its
// four sub-steps, fetches a quarter of step kt+h+2 into stage h and decodes+
// stores a quarter of stage 1-h into buffer 1-h, then synchronizes.  Spread
// this way, the loads of a step do not queue up behind each other at its
// start.  Fetch indices are clamped to the last step, so the tail re-reads
// (in bounds) data it never uses.
template <class C, bool F16, class SA, class SB, class FetchA, class FetchB, class StoreA, class StoreB>
__device__ __forceinline__ void k_loop(int nk, uint4 (*As)[C::BM * 8], uint4 (*Bs)[C::BN * 8],
                                       f32x16 (&acc)[C::MI][C::NI], int wm, int wn, int lane, FetchA fa,
                                       FetchB fb, StoreA sta, StoreB stb) {
  // Steps are processed in pairs; an odd count gets one all-zero step (its
  // blocks are past the end of K), so the loop body has no exit in between.
  SA s0, s1;
  SB t0, t1;
  fa(s0, 0, -1);
  fb(t0, 0, -1);
  fa(s1, 1, -1);
  fb(t1, 1, -1);
#pragma unroll
  for (int part = 0; part < 4; ++part) {
    sta(s0, As[0], part);
    stb(t0, Bs[0], part);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    mfma_step<C, F16>(As[0], Bs[0], acc, wm, wn, lane, [&](int part) {
      fa(s0, kt + 2, part);
      fb(t0, kt + 2, part);
      sta(s1, As[1], part);
      stb(t1, Bs[1], part);
    });
    __syncthreads();
    mfma_step<C, F16>(As[1], Bs[1], acc, wm, wn, lane, [&](int part) {
      fa(s1, kt + 3, part);
      fb(t1, kt + 3, part);
      sta(s0, As[0], part);
      stb(t0, Bs[0], part);
    });
    __syncthreads();
  }
}

// Map this workgroup to (expert e, rows [m0, min(m0+BM, mend)), n-tile nt).
// The grid is an upper bound of the tile count (ragged experts); the real
// count T comes from the tile list (or, for one expert, from its row range)
// and is split into 8 contiguous ranges of ceil(T/8) tiles, range x on XCD x
// (= blockIdx % 8), so every XCD gets the same share of real tiles and keeps
// consecutive tiles (the n-tiles of one m-tile, then the m-tiles of one
// expert) in its own L2.  Returns false for surplus workgroups (uniformly
// for the whole workgroup).  One expert (a dense GEMM) needs no tile list.
template <class C>
__device__ __forceinline__ bool tile_setup(const Params &p, int &nt, int &e, int &m0, int &mend, int &s_e, int &s_m0,
                                           int &s_mend) {
  int lo = 0, hi = 0, mtiles;
  if (p.E == 1) {
    lo = p.expert_offsets[0];
    hi = p.expert_offsets[1];
    mtiles = hi > lo ? (hi - lo + C::BM - 1) / C::BM : 0;
  } else {
    mtiles = p.tile_offsets[p.E];
  }
  const int per_xcd = (mtiles * p.n_tiles + 7) / 8;
  const int j = blockIdx.x >> 3;
  if (j >= per_xcd) return false;
  const int logical = (blockIdx.x & 7) * per_xcd + j;
  const int mt = logical / p.n_tiles;
  nt = logical % p.n_tiles;
  if (mt >= mtiles) return false;
  if (p.E == 1) {
    e = 0;
    m0 = lo + mt * C::BM;
    mend = hi;
    return true;
  }
  if (threadIdx.x == 0) {
    int l = 0, h = p.E;  // largest e with tile_offsets[e] <= mt (skips empty experts)
    while (h - l > 1) {
      const int mid = (l + h) >> 1;
      if (p.tile_offsets[mid] <= mt) l = mid; else h = mid;
    }
    s_e = l;
    s_m0 = p.expert_offsets[l] + (mt - p.tile_offsets[l]) * C::BM;
    s_mend = p.expert_offsets[l + 1];
  }
  __syncthreads();
  e = s_e;
  m0 = s_m0;
  mend = s_mend;
  return true;
}

// Scale, optional SwiGLU, and store one wave's accumulators.
template <class C, int MODE, int EPI, bool HAS_RES, bool TRANS = false>
__device__ __forceinline__ float epilogue(const Params &p, f32x16 (&acc)[C::MI][C::NI], int e, int m0, int mend,
                                          int nt, int wm, int wn, int lane, float *stage = nullptr) {
  float hmax = 0.0f;  // largest |stored bf16 value| (NaN skipped), for the output's tensor scale
  float ascale = 1.0f;
  if constexpr (MODE == 0) ascale = HAS_RES ? *p.r_g : *p.x_g;
  if constexpr (MODE == 2) ascale = *p.x_g;
  if constexpr (TRANS) {
    // Accumulators hold Y transposed (see mfmas): four consecutive columns
    // per register group, stored as one 16-byte (FP32) or 8-byte (bf16)
    // vector.  Segments and SwiGLU halves are multiples of 32 columns, so a
    // group never straddles them.
    if constexpr (EPI == 0) {
      // Through this wave's LDS stage, one 32-row block (mi) at a time: the
      // scaled accumulators go in as 16-byte row pieces (rows padded by 16
      // bytes so the 32 rows of a write fall in distinct banks), and come
      // back out as whole row segments, TN/4 lanes per row, so each store
      // instruction writes 64/(TN/4) full segments of TN columns.
      const int64_t seg_len = p.N / p.n_seg;
      constexpr int RS = C::TN + 4;         // floats per staged row
      constexpr int LPR = C::TN / 4;        // lanes per row on the way out
      constexpr int RPI = 64 / LPR;         // rows per store instruction
      const int64_t col0 = static_cast<int64_t>(nt) * C::BN + wn * C::TN;
      float sc[C::NI][4];
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sc[ni][j] = ascale;
          if constexpr (MODE < 3 && MODE != 1)
            sc[ni][j] = p.w_g[e * p.n_seg + (col0 + ni * 32 + 8 * j + 4 * (lane >> 5)) / seg_len] * ascale;
        }
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(stage + (lane & 31) * RS + ni * 32 + 8 * j + 4 * (lane >> 5)) =
                make_float4(acc[mi][ni][4 * j] * sc[ni][j], acc[mi][ni][4 * j + 1] * sc[ni][j],
                            acc[mi][ni][4 * j + 2] * sc[ni][j], acc[mi][ni][4 * j + 3] * sc[ni][j]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
          const int r = t * RPI + lane / LPR, c4 = (lane % LPR) * 4;
          const float4 v = *reinterpret_cast<const float4 *>(stage + r * RS + c4);
          const int i = m0 + wm * C::TM + mi * 32 + r;
          if (i < mend) {
            const int64_t at = static_cast<int64_t>(i) * p.N + col0 + c4;
            if (p.y_bf16) {
              const uint32_t h0 = f32_to_bf16_bits(v.x), h1 = f32_to_bf16_bits(v.y), h2b = f32_to_bf16_bits(v.z),
                             h3 = f32_to_bf16_bits(v.w);
              hmax = fmaxf(fmaxf(fmaxf(hmax, fabsf(bf16_bits_to_f32(h0))), fabsf(bf16_bits_to_f32(h1))),
                           fmaxf(fabsf(bf16_bits_to_f32(h2b)), fabsf(bf16_bits_to_f32(h3))));
              *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + at) = make_uint2(h0 | (h1 << 16), h2b | (h3 << 16));
            } else {  // FP32 y leaves as a stream (a later kernel reads it back from HBM)
              typedef float f32x4_nt __attribute__((ext_vector_type(4)));
              const f32x4_nt t = {v.x, v.y, v.z, v.w};
              __builtin_nontemporal_store(t, reinterpret_cast<f32x4_nt *>(static_cast<float *>(p.y) + at));
            }
          }
        }
      }
    } else {
      static_assert(EPI == 0 || C::NI % 2 == 0, "SWIGLU needs an even number of 32-column tiles per wave");
      const int64_t I = p.N / 2;
      float sg = ascale, su = ascale;
      if constexpr (MODE < 3 && MODE != 1) {
        sg = p.w_g[e * 2] * ascale;
        su = p.w_g[e * 2 + 1] * ascale;
      }
#pragma unroll
      for (int ni = 0; ni < C::NI / 2; ++ni)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col =
              static_cast<int64_t>(nt) * (C::BN / 2) + wn * (C::TN / 2) + ni * 32 + 8 * j + 4 * (lane >> 5);
#pragma unroll
          for (int mi = 0; mi < C::MI; ++mi) {
            const int i = m0 + wm * C::TM + mi * 32 + (lane & 31);
            if (i < mend) {
              uint32_t hb[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const float g = acc[mi][ni][4 * j + u] * sg;
                const float up = acc[mi][ni + C::NI / 2][4 * j + u] * su;
                hb[u] = f32_to_bf16_bits(silu(g) * up);
                hmax = fmaxf(hmax, fabsf(bf16_bits_to_f32(hb[u])));
              }
              *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + static_cast<int64_t>(i) * I + col) =
                  make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            }
          }
        }
    }
    return hmax;
  }
  if constexpr (EPI == 0) {
    const int64_t seg_len = p.N / p.n_seg;
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      const int64_t col = static_cast<int64_t>(nt) * C::BN + wn * C::TN + ni * 32 + (lane & 31);
      float sc = ascale;
      if constexpr (MODE < 3 && MODE != 1) sc = p.w_g[e * p.n_seg + col / seg_len] * ascale;
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = m0 + wm * C::TM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (i < mend) {
            const float v = acc[mi][ni][r] * sc;
            if (p.y_bf16) {
              const uint32_t hb = f32_to_bf16_bits(v);
              static_cast<uint16_t *>(p.y)[static_cast<int64_t>(i) * p.N + col] = static_cast<uint16_t>(hb);
              hmax = fmaxf(hmax, fabsf(bf16_bits_to_f32(hb)));
            } else {
              __builtin_nontemporal_store(v, static_cast<float *>(p.y) + static_cast<int64_t>(i) * p.N + col);
            }
          }
        }
    }
  } else {
    static_assert(EPI == 0 || C::NI % 2 == 0, "SWIGLU needs an even number of 32-column tiles per wave");
    const int64_t I = p.N / 2;
    float sg = ascale, su = ascale;
    if constexpr (MODE < 3 && MODE != 1) {
      sg = p.w_g[e * 2] * ascale;
      su = p.w_g[e * 2 + 1] * ascale;
    }
#pragma unroll
    for (int ni = 0; ni < C::NI / 2; ++ni) {
      const int64_t col = static_cast<int64_t>(nt) * (C::BN / 2) + wn * (C::TN / 2) + ni * 32 + (lane & 31);
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = m0 + wm * C::TM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (i < mend) {
            const float g = acc[mi][ni][r] * sg;
            const float u = acc[mi][ni + C::NI / 2][r] * su;
            const uint32_t hb = f32_to_bf16_bits(silu(g) * u);
            static_cast<uint16_t *>(p.y)[static_cast<int64_t>(i) * I + col] = static_cast<uint16_t>(hb);
            hmax = fmaxf(hmax, fabsf(bf16_bits_to_f32(hb)));
          }
        }
    }
  }
  return hmax;
}

// MODE 0: NVFP4 operands (+ residual segment if HAS_RES), fp16 MFMA;
// MODE 1: bf16 operands, bf16 MFMA;
// MODE 2: the RAC-merged fp16 activation (X' + (gr/gx) R', built by the GEMM
// prepare step) times NVFP4 weights, fp16 MFMA over K alone;
// MODE 3: bf16 activations times bf16 master weights fake-quantized in
// registers (the trainer's W4A16 forward with the QDQ fused), bf16 MFMA;
// MODE 4: bf16 activations times NVFP4 weights decoded to their QDQ bf16
// values on the way into LDS (the same forward, W_qdq never written), bf16
// MFMA.
template <class C, int MODE, int EPI, bool HAS_RES>
__global__ __launch_bounds__(C::THREADS, C::MINB) void k_gemm(Params p) {
  __shared__ uint4 As[2][C::BM * 8];
  __shared__ uint4 Bs[2][C::BN * 8];
  __shared__ int s_e, s_m0, s_mend;

  int nt, e, m0, mend;
  if (!tile_setup<C>(p, nt, e, m0, mend, s_e, s_m0, s_mend)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;

  auto act_row = [&](int r) -> int64_t {
    int i = m0 + r;
    if (i >= mend) i = mend - 1;  // padding rows re-read a valid row; never stored
    return p.row_token ? static_cast<int64_t>(p.row_token[i]) : static_cast<int64_t>(i);
  };

  f32x16 acc[C::MI][C::NI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int64_t wbase = static_cast<int64_t>(e) * p.N;  // expert's first weight row
  constexpr int T = C::THREADS;

  if constexpr (MODE == 0) {
    const int nblk = static_cast<int>(p.K / 16);
    int64_t arow[C::FA], abase[C::FA], bbase[C::FB];
#pragma unroll
    for (int q = 0; q < C::FA; ++q) {
      arow[q] = act_row(fp4_row(threadIdx.x) + q * (T / 4));
      abase[q] = arow[q] * nblk;
    }
#pragma unroll
    for (int q = 0; q < C::FB; ++q)
      bbase[q] = (wbase + w_row_of<C, EPI>(fp4_row(threadIdx.x) + q * (T / 4), nt, p.N)) * nblk;
    // activation and this expert's weights as buffer resources
    const int64_t wrows = p.N;
    const auto xc = buf_rsrc(p.x_codes, p.act_rows * (p.K / 2)), xs = buf_rsrc(p.x_scales, p.act_rows * nblk);
    const auto wc = buf_rsrc(p.w_codes + wbase * (p.K / 2), wrows * (p.K / 2));
    const auto ws = buf_rsrc(p.w_scales + wbase * nblk, wrows * nblk);
    uint32_t ablk[C::FA], bblk[C::FB];
#pragma unroll
    for (int q = 0; q < C::FA; ++q) ablk[q] = static_cast<uint32_t>(abase[q] + (threadIdx.x & 3));
#pragma unroll
    for (int q = 0; q < C::FB; ++q) bblk[q] = static_cast<uint32_t>(bbase[q] - wbase * nblk + (threadIdx.x & 3));
    k_loop<C, true, Fp4Stage<C::FA>, Fp4Stage<C::FB>>(
        static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
        [&](Fp4Stage<C::FA> &st, int kt, int part) { fp4_fetch_buf(st, xc, xs, ablk, nblk, kt, part); },
        [&](Fp4Stage<C::FB> &st, int kt, int part) { fp4_fetch_buf(st, wc, ws, bblk, nblk, kt, part); },
        [&](const Fp4Stage<C::FA> &st, uint4 *tile, int part) { fp4_store<C::FA, T>(st, tile, part); },
        [&](const Fp4Stage<C::FB> &st, uint4 *tile, int part) { fp4_store<C::FB, T>(st, tile, part); });
    if constexpr (HAS_RES) {
      const float ratio = *p.x_g / *p.r_g;
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ratio;
      const int rblk = static_cast<int>(p.kpad / 16);
      int64_t rbase[C::FA], gbase[C::HB];
#pragma unroll
      for (int q = 0; q < C::FA; ++q) rbase[q] = arow[q] * rblk;
#pragma unroll
      for (int q = 0; q < C::HB; ++q)
        gbase[q] = (wbase + w_row_of<C, EPI>((threadIdx.x >> 3) + q * (T / 8), nt, p.N)) * p.kpad;
      k_loop<C, true, Fp4Stage<C::FA>, RawStage<C::HB>>(
          static_cast<int>((p.kpad + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
          [&](Fp4Stage<C::FA> &st, int kt, int part) { fp4_fetch(st, p.r_codes, p.r_scales, rbase, rblk, kt, part); },
          [&](RawStage<C::HB> &st, int kt, int part) { raw_fetch(st, p.wg_f16, gbase, static_cast<int>(p.kpad), kt, part); },
          [&](const Fp4Stage<C::FA> &st, uint4 *tile, int part) { fp4_store<C::FA, T>(st, tile, part); },
          [&](const RawStage<C::HB> &st, uint4 *tile, int part) { raw_store<C::HB, T>(st, tile, part); });
    }
  } else if constexpr (MODE == 2) {
    const int nblk = static_cast<int>(p.K / 16);
    int64_t abase[C::HA], bbase[C::FB];
#pragma unroll
    for (int q = 0; q < C::HA; ++q) abase[q] = act_row((threadIdx.x >> 3) + q * (T / 8)) * p.K;
#pragma unroll
    for (int q = 0; q < C::FB; ++q)
      bbase[q] = (wbase + w_row_of<C, EPI>(fp4_row(threadIdx.x) + q * (T / 4), nt, p.N)) * nblk;
    const auto xa = buf_rsrc(p.x_f16, p.act_rows * p.K * 2);
    const auto wc = buf_rsrc(p.w_codes + wbase * (p.K / 2), p.N * (p.K / 2));
    const auto ws = buf_rsrc(p.w_scales + wbase * nblk, p.N * nblk);
    uint32_t aofs[C::HA], bblk[C::FB];
#pragma unroll
    for (int q = 0; q < C::HA; ++q) aofs[q] = static_cast<uint32_t>(2 * (abase[q] + (threadIdx.x & 7) * 8));
#pragma unroll
    for (int q = 0; q < C::FB; ++q) bblk[q] = static_cast<uint32_t>(bbase[q] - wbase * nblk + (threadIdx.x & 3));
    k_loop<C, true, RawStage<C::HA>, Fp4Stage<C::FB>>(
        static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
        [&](RawStage<C::HA> &st, int kt, int part) { raw_fetch_buf(st, xa, aofs, static_cast<int>(p.K), kt, part); },
        [&](Fp4Stage<C::FB> &st, int kt, int part) { fp4_fetch_buf(st, wc, ws, bblk, nblk, kt, part); },
        [&](const RawStage<C::HA> &st, uint4 *tile, int part) { raw_store<C::HA, T, false>(st, tile, part); },
        [&](const Fp4Stage<C::FB> &st, uint4 *tile, int part) { fp4_store<C::FB, T>(st, tile, part); });
  } else if constexpr (MODE == 4) {
    const int nblk = static_cast<int>(p.K / 16);
    int64_t abase[C::HA], bbase[C::FB];
    float gq[C::FB];
#pragma unroll
    for (int q = 0; q < C::HA; ++q) abase[q] = act_row((threadIdx.x >> 3) + q * (T / 8)) * p.K;
#pragma unroll
    for (int q = 0; q < C::FB; ++q) {
      const int64_t wr = w_row_of<C, EPI>(fp4_row(threadIdx.x) + q * (T / 4), nt, p.N);
      bbase[q] = (wbase + wr) * nblk;
      gq[q] = w_scale_of(p, e, wr);
    }
    k_loop<C, false, RawStage<C::HA>, Fp4Stage<C::FB>>(
        static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
        [&](RawStage<C::HA> &st, int kt, int part) { raw_fetch(st, p.x_bf16, abase, static_cast<int>(p.K), kt, part); },
        [&](Fp4Stage<C::FB> &st, int kt, int part) { fp4_fetch(st, p.w_codes, p.w_scales, bbase, nblk, kt, part); },
        [&](const RawStage<C::HA> &st, uint4 *tile, int part) { raw_store<C::HA, T>(st, tile, part); },
        [&](const Fp4Stage<C::FB> &st, uint4 *tile, int part) { fp4_qdq_store<C::FB, T>(st, tile, part, gq); });
  } else if constexpr (MODE == 3) {
    int64_t abase[C::HA], bbase[C::HB];
    TensorScale gq[C::HB];
#pragma unroll
    for (int q = 0; q < C::HA; ++q) abase[q] = act_row((threadIdx.x >> 3) + q * (T / 8)) * p.K;
#pragma unroll
    for (int q = 0; q < C::HB; ++q) {
      const int64_t wr = w_row_of<C, EPI>((threadIdx.x >> 3) + q * (T / 8), nt, p.N);
      bbase[q] = (wbase + wr) * p.K;
      gq[q] = tensor_scale(w_scale_of(p, e, wr));
    }
    k_loop<C, false, RawStage<C::HA>, RawStage<C::HB>>(
        static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
        [&](RawStage<C::HA> &st, int kt, int part) { raw_fetch(st, p.x_bf16, abase, static_cast<int>(p.K), kt, part); },
        [&](RawStage<C::HB> &st, int kt, int part) { raw_fetch(st, p.w_bf16, bbase, static_cast<int>(p.K), kt, part); },
        [&](const RawStage<C::HA> &st, uint4 *tile, int part) { raw_store<C::HA, T>(st, tile, part); },
        [&](const RawStage<C::HB> &st, uint4 *tile, int part) { qdq_store<C::HB, T>(st, tile, part, gq); });
  } else {
    int64_t abase[C::HA], bbase[C::HB];
#pragma unroll
    for (int q = 0; q < C::HA; ++q) abase[q] = act_row((threadIdx.x >> 3) + q * (T / 8)) * p.K;
#pragma unroll
    for (int q = 0; q < C::HB; ++q) bbase[q] = (wbase + w_row_of<C, EPI>((threadIdx.x >> 3) + q * (T / 8), nt, p.N)) * p.K;
    k_loop<C, false, RawStage<C::HA>, RawStage<C::HB>>(
        static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, wm, wn, lane,
        [&](RawStage<C::HA> &st, int kt, int part) { raw_fetch(st, p.x_bf16, abase, static_cast<int>(p.K), kt, part); },
        [&](RawStage<C::HB> &st, int kt, int part) { raw_fetch(st, p.w_bf16, bbase, static_cast<int>(p.K), kt, part); },
        [&](const RawStage<C::HA> &st, uint4 *tile, int part) { raw_store<C::HA, T>(st, tile, part); },
        [&](const RawStage<C::HB> &st, uint4 *tile, int part) { raw_store<C::HB, T>(st, tile, part); });
  }

  // Per-wave epilogue stages in the operand tiles (free after the last step):
  // half the waves in As, half in Bs.
  constexpr int kWaves = C::THREADS / 64, kPerArr = kWaves / 2;
  static_assert(kPerArr * 32 * (C::TN + 4) * 4 <= static_cast<int>(sizeof(As)) &&
                    kPerArr * 32 * (C::TN + 4) * 4 <= static_cast<int>(sizeof(Bs)),
                "epilogue stages fit in the operand tiles");
  float *stage = reinterpret_cast<float *>(wave < kPerArr ? &As[0][0] : &Bs[0][0]) + (wave % kPerArr) * 32 * (C::TN + 4);
  const float hmax = epilogue<C, MODE, EPI, HAS_RES, true>(p, acc, e, m0, mend, nt, wm, wn, lane, stage);
  if (p.amax_ws != nullptr) amax_gather(p.amax_ws, hmax);
}

// ---- 8-wave ping-pong kernel for 256x256 tiles ------------------------------
// The eight waves form two groups of four (one wave of each group per SIMD):
// group g owns output rows [128g, 128g+128) and stages rows [128g, 128g+128)
// of both the A and the B tile.  The groups run a phase apart: while one group
// issues MFMAs on the current LDS buffer, the other decodes and stores its half
// of the next K step and issues the global loads for the step after, so the
// matrix core of every SIMD always has one wave feeding it.  Each K step is
// two phases separated by barriers:
//   phase 1: group 0 computes step k | group 1 stores its half of step k+1
//   phase 2: group 0 stores its half of step k+1 | group 1 computes step k
// Two LDS buffers suffice: buffer (k+1)%2 was last read by group 0 in phase 1
// and by group 1 in phase 2 of step k-1, both before either group writes it in
// step k, and both halves of step k+1 are written before phase 1 of step k+1.
using CfgPP = Cfg<256, 256, 2, 4, 1>;

template <int P>
__device__ __forceinline__ void fp4_store_rows(const Fp4Stage<P> &st, uint4 *tile, const int (&rows)[P]) {
  const int c = (threadIdx.x & 3) * 2;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const h2 sc = scale_h2(st.ok ? st.s[p] : 0u);
    tile[swz(rows[p], c)] = decode8_f16(st.w[p].x, sc);
    tile[swz(rows[p], c + 1)] = decode8_f16(st.w[p].y, sc);
  }
}

template <int P>
__device__ __forceinline__ void raw_store_rows(const RawStage<P> &st, uint4 *tile, const int (&rows)[P]) {
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int q = 0; q < P; ++q) tile[swz(rows[q], c)] = st.ok ? st.v[q] : make_uint4(0, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ void pp_compute(const uint4 *As, const uint4 *Bs, f32x16 (&acc)[CfgPP::MI][CfgPP::NI],
                                           int wm, int wn, int lane) {
  __builtin_amdgcn_s_setprio(1);
  mfma_step<CfgPP, F16>(As, Bs, acc, wm, wn, lane, [](int) {});
  __builtin_amdgcn_s_setprio(0);
}

// init(): fetch step 0, store it into buffer 0, fetch step 1.
// mem(k, buf): store this thread's part of step k+1 into buffer buf, fetch step k+2.
template <bool F16, class Init, class Mem>
__device__ __forceinline__ void pp_loop(int nk, uint4 (*As)[CfgPP::BM * 8], uint4 (*Bs)[CfgPP::BN * 8],
                                        f32x16 (&acc)[CfgPP::MI][CfgPP::NI], int g, int wm, int wn, int lane,
                                        Init init, Mem mem) {
  init();
  __syncthreads();
  for (int k = 0; k < nk; ++k) {
    const int cur = k & 1;
    if (g == 0)
      pp_compute<F16>(As[cur], Bs[cur], acc, wm, wn, lane);
    else
      mem(k, cur ^ 1);
    __syncthreads();
    if (g == 0)
      mem(k, cur ^ 1);
    else
      pp_compute<F16>(As[cur], Bs[cur], acc, wm, wn, lane);
    __syncthreads();
  }
}

template <int MODE, int EPI, bool HAS_RES>
__global__ __launch_bounds__(CfgPP::THREADS, 1) void k_gemm_pp(Params p) {
  using C = CfgPP;
  __shared__ uint4 As[2][C::BM * 8];
  __shared__ uint4 Bs[2][C::BN * 8];
  __shared__ int s_e, s_m0, s_mend;
  int nt, e, m0, mend;
  if (!tile_setup<C>(p, nt, e, m0, mend, s_e, s_m0, s_mend)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = wave >> 2, wm = g, wn = wave & 3;
  const int tg = threadIdx.x & 255;

  auto act_row = [&](int r) -> int64_t {
    int i = m0 + r;
    if (i >= mend) i = mend - 1;  // padding rows re-read a valid row; never stored
    return p.row_token ? static_cast<int64_t>(p.row_token[i]) : static_cast<int64_t>(i);
  };

  f32x16 acc[C::MI][C::NI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int64_t wbase = static_cast<int64_t>(e) * p.N;

  if constexpr (MODE == 0) {
    const int nblk = static_cast<int>(p.K / 16);
    int arows[2];
    int64_t arow[2], abase[2], bbase[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      arows[q] = g * 128 + fp4_row(tg) + q * 64;
      arow[q] = act_row(arows[q]);
      abase[q] = arow[q] * nblk;
      bbase[q] = (wbase + w_row_of<C, EPI>(arows[q], nt, p.N)) * nblk;
    }
    Fp4Stage<2> sa, sb;
    auto fetch = [&](int kt) {
      fp4_fetch(sa, p.x_codes, p.x_scales, abase, nblk, kt);
      fp4_fetch(sb, p.w_codes, p.w_scales, bbase, nblk, kt);
    };
    auto store = [&](int buf) {
      fp4_store_rows(sa, As[buf], arows);
      fp4_store_rows(sb, Bs[buf], arows);
    };
    pp_loop<true>(static_cast<int>((p.K + BK - 1) / BK), As, Bs, acc, g, wm, wn, lane,
                  [&] { fetch(0); store(0); fetch(1); },
                  [&](int k, int buf) { store(buf); fetch(k + 2); });
    if constexpr (HAS_RES) {
      const float ratio = *p.x_g / *p.r_g;
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ratio;
      const int rblk = static_cast<int>(p.kpad / 16);
      const int kpad = static_cast<int>(p.kpad);
      int64_t rbase[2], gbase[4];
      int grows[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) rbase[q] = arow[q] * rblk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        grows[q] = g * 128 + (tg >> 3) + q * 32;
        gbase[q] = (wbase + w_row_of<C, EPI>(grows[q], nt, p.N)) * p.kpad;
      }
      Fp4Stage<2> sr;
      RawStage<4> sg;
      auto rfetch = [&](int kt) {
        fp4_fetch(sr, p.r_codes, p.r_scales, rbase, rblk, kt);
        raw_fetch(sg, p.wg_f16, gbase, kpad, kt);
      };
      auto rstore = [&](int buf) {
        fp4_store_rows(sr, As[buf], arows);
        raw_store_rows(sg, Bs[buf], grows);
      };
      pp_loop<true>((kpad + BK - 1) / BK, As, Bs, acc, g, wm, wn, lane,
                    [&] { rfetch(0); rstore(0); rfetch(1); },
                    [&](int k, int buf) { rstore(buf); rfetch(k + 2); });
    }
  } else if constexpr (MODE == 4) {
    const int K = static_cast<int>(p.K);
    const int nblk = K / 16;
    int arows[4], brows[2];
    int64_t abase[4], bbase[2];
    float gq[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      arows[q] = g * 128 + (tg >> 3) + q * 32;
      abase[q] = act_row(arows[q]) * p.K;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      brows[q] = g * 128 + fp4_row(tg) + q * 64;
      const int64_t wr = w_row_of<C, EPI>(brows[q], nt, p.N);
      bbase[q] = (wbase + wr) * nblk;
      gq[q] = w_scale_of(p, e, wr);
    }
    RawStage<4> sa;
    Fp4Stage<2> sb;
    auto fetch = [&](int kt) __attribute__((always_inline)) {
      raw_fetch(sa, p.x_bf16, abase, K, kt);
      fp4_fetch(sb, p.w_codes, p.w_scales, bbase, nblk, kt);
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
      raw_store_rows(sa, As[buf], arows);
      const int c = (tg & 3) * 2;
      uint4 c0, c1;
      qdq_decode16(sb.w[0], sb.s[0], gq[0], sb.ok, c0, c1);
      Bs[buf][swz(brows[0], c)] = c0;
      Bs[buf][swz(brows[0], c + 1)] = c1;
      qdq_decode16(sb.w[1], sb.s[1], gq[1], sb.ok, c0, c1);
      Bs[buf][swz(brows[1], c)] = c0;
      Bs[buf][swz(brows[1], c + 1)] = c1;
    };
    pp_loop<false>((K + BK - 1) / BK, As, Bs, acc, g, wm, wn, lane,
                   [&]() __attribute__((always_inline)) { fetch(0); store(0); fetch(1); },
                   [&](int k, int buf) __attribute__((always_inline)) { store(buf); fetch(k + 2); });
  } else {
    const int K = static_cast<int>(p.K);
    int arows[4];
    int64_t abase[4], bbase[4];
    TensorScale gq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      arows[q] = g * 128 + (tg >> 3) + q * 32;
      abase[q] = act_row(arows[q]) * p.K;
      const int64_t wr = w_row_of<C, EPI>(arows[q], nt, p.N);
      bbase[q] = (wbase + wr) * p.K;
      gq[q] = tensor_scale(MODE == 3 ? w_scale_of(p, e, wr) : 1.0f);
    }
    RawStage<4> sa, sb;
    // The lambdas are forced inline: with the QDQ body they exceed the
    // inliner's budget, and a lambda left as a call keeps the arrays it
    // captures by reference in scratch memory.
    auto fetch = [&](int kt) __attribute__((always_inline)) {
      raw_fetch(sa, p.x_bf16, abase, K, kt);
      raw_fetch(sb, p.w_bf16, bbase, K, kt);
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
      raw_store_rows(sa, As[buf], arows);
      if constexpr (MODE == 3) {
        const int c = threadIdx.x & 7;
        Bs[buf][swz(arows[0], c)] = qdq_chunk(sb.v[0], sb.ok, gq[0]);
        Bs[buf][swz(arows[1], c)] = qdq_chunk(sb.v[1], sb.ok, gq[1]);
        Bs[buf][swz(arows[2], c)] = qdq_chunk(sb.v[2], sb.ok, gq[2]);
        Bs[buf][swz(arows[3], c)] = qdq_chunk(sb.v[3], sb.ok, gq[3]);
      } else {
        raw_store_rows(sb, Bs[buf], arows);
      }
    };
    pp_loop<false>((K + BK - 1) / BK, As, Bs, acc, g, wm, wn, lane,
                   [&]() __attribute__((always_inline)) { fetch(0); store(0); fetch(1); },
                   [&](int k, int buf) __attribute__((always_inline)) { store(buf); fetch(k + 2); });
  }
  // per-wave epilogue stages in the operand tiles, free after the last step
  float *stage = reinterpret_cast<float *>(wave < 4 ? &As[0][0] : &Bs[0][0]) + (wave % 4) * 32 * (C::TN + 4);
  epilogue<C, MODE, EPI, HAS_RES, true>(p, acc, e, m0, mend, nt, wm, wn, lane, stage);
}

// ---- DMA-staged NVFP4 kernel (128 x 64NI tiles, 8 waves) ---------------------
// Operands travel from global memory to LDS as raw codes and scales
// (global_load_lds, no registers on the way), so an LDS stage is a quarter of
// the size of a decoded fp16 tile.  Each wave decodes its own MFMA fragments
// from LDS (cvt + pk_mul, exact).
//
// The eight waves form two groups of four; both groups cover the whole
// output tile (64 x 32NI per wave) and split every K step between them, so a
// tile keeps two waves per SIMD busy.  The two partial accumulators are
// summed through LDS at the end.  NI = 2 (128x128, two workgroups per CU) or
// NI = 3 (128x192, one per CU).
//
// A main-segment K step is 128 elements: 64 code bytes (four 16-byte chunks)
// and 8 scale bytes per row.  The contraction order inside a step is
// permuted identically for both operands: in group g, lane half h of a
// fragment takes chunk 2g+h of its row (one ds_read_b128 holding the 8 codes
// of each of 4 MFMA sub-steps) and its two block scales.  The residual
// segment (extended K) has 64-element steps: 32 code bytes and 4 scale bytes
// per residual row, 128 bytes of gathered fp16 weight columns per weight row;
// in group g, lane half h takes the 16 residual codes [32h + 16g, +16).
// Stage k+2 is in flight while step k is computed; one barrier per step.
// Every wave issues the same number of DMA instructions (P) per step in both
// segments (a few duplicate loads write identical bytes to the same LDS words
// to even the count), so "all but the newest P" is the wait for the step
// about to be computed.
namespace dmak {

constexpr int kThreads = 512;
constexpr int kStages = 3;
constexpr int kStepM = 128;  // main-segment K step
constexpr int kStepR = 64;   // residual-segment K step

template <int NI_>
struct Lay {
  static constexpr int NI = NI_;
  static constexpr int BM = 128, BN = 64 * NI;
  using C = Cfg<BM, BN, 2, 2, NI == 2 ? 2 : 1>;  // per-group wave layout: tile_setup, w_row_of, epilogue
  static constexpr int P = NI == 2 ? 3 : 4;  // DMA instructions per wave per step
  // Main stage (bytes): A codes [128][64], B codes [BN][64], A scales [128][8], B scales [BN][8].
  static constexpr int MA = 0, MB = 8192, MAS = MB + BN * 64, MBS = MAS + 1024, MEND = MBS + BN * 8;
  // Residual stage: R codes [128][32], R scales [128][4], gathered W [BN][128 B].
  static constexpr int RA = 0, RAS = 4096, RB = 4608, REND = RB + BN * 128;
  // Merged stage (64-element steps): merged fp16 activation [128][128 B],
  // W codes [BN][32], W scales [BN][4].
  static constexpr int XA = 0, XB = 16384, XBS = XB + BN * 32, XEND = XBS + BN * 4;
  static constexpr int STAGE0 = MEND > REND ? MEND : REND;
  static constexpr int STAGE = STAGE0 > XEND ? STAGE0 : XEND;
};

// DMA staging helpers (dma, wait_vm, barrier_no_fence): dma.hpp.
template <int P>
__device__ __forceinline__ void wait_all_but_one_step() {
  wait_vm<P>();
}
__device__ __forceinline__ void wait_all() { wait_vm<0>(); }

// Chunk slot swizzles (16-byte units) that make the fragment reads
// bank-conflict-free: 64-byte rows, 32-byte rows, 128-byte rows.
__device__ __forceinline__ int slot64(int row, int c) { return c ^ ((row >> 2) & 3); }
__device__ __forceinline__ int slot32(int row, int c) { return c ^ ((row >> 3) & 1); }
__device__ __forceinline__ int slot128(int row, int c) { return c ^ ((row >> 1) & 7); }

// (dec(s), dec(s)) for bytes `sel` (two bytes of a scale word, each doubled).
__device__ __forceinline__ void scales2(uint32_t w, uint32_t sel, h2 (&s)[2]) {
  const uint32_t d = __builtin_amdgcn_perm(w, w, sel);
  s[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false);
  s[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true);
}

template <int NI>
__device__ __forceinline__ void mfmas(const uint4 (&a)[2], const uint4 (&b)[NI], f32x16 (&acc)[2][NI]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a[mi]), __builtin_bit_cast(h8, b[ni]),
                                                           acc[mi][ni], 0, 0, 0);
}

// Group g's half of one main step from stage `st`: 4 sub-steps of 2*NI MFMAs.
template <int NI>
__device__ __forceinline__ void compute_main(const uint8_t *st, f32x16 (&acc)[2][NI], int wm, int wn, int g,
                                             int lane) {
  using L = Lay<NI>;
  const int r = lane & 31, h = lane >> 5, c = 2 * g + h;
  const uint32_t sel = h ? 0x03030202u : 0x01010000u;  // blocks 4g+2h, 4g+2h+1 of the row's 8
  uint4 ca[2], cb[NI];
  h2 sa[2][2], sb[NI][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + i * 32 + r;
    scales2(*reinterpret_cast<const uint32_t *>(st + L::MAS + row * 8 + 4 * g), sel, sa[i]);
    ca[i] = *reinterpret_cast<const uint4 *>(st + L::MA + row * 64 + slot64(row, c) * 16);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = wn * 32 * NI + i * 32 + r;
    scales2(*reinterpret_cast<const uint32_t *>(st + L::MBS + row * 8 + 4 * g), sel, sb[i]);
    cb[i] = *reinterpret_cast<const uint4 *>(st + L::MB + row * 64 + slot64(row, c) * 16);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 a[2], b[NI];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t wa[4] = {ca[i].x, ca[i].y, ca[i].z, ca[i].w};
      a[i] = decode8_f16(wa[j], sa[i][j >> 1]);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t wb[4] = {cb[i].x, cb[i].y, cb[i].z, cb[i].w};
      b[i] = decode8_f16(wb[j], sb[i][j >> 1]);
    }
    mfmas<NI>(a, b, acc);
  }
}

// Group g's half of one residual step: 2 sub-steps; A = residual codes, B =
// gathered fp16 weight columns.
template <int NI>
__device__ __forceinline__ void compute_res(const uint8_t *st, f32x16 (&acc)[2][NI], int wm, int wn, int g,
                                            int lane) {
  using L = Lay<NI>;
  const int r = lane & 31, h = lane >> 5;
  uint2 ca[2];
  h2 sa[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + i * 32 + r;
    ca[i] = *reinterpret_cast<const uint2 *>(st + L::RA + row * 32 + slot32(row, h) * 16 + 8 * g);
    sa[i] = scale_h2(st[L::RAS + row * 4 + 2 * h + g]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint4 a[2], b[NI];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = decode8_f16(j ? ca[i].y : ca[i].x, sa[i]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = wn * 32 * NI + i * 32 + r;
      b[i] = *reinterpret_cast<const uint4 *>(st + L::RB + row * 128 + slot128(row, 4 * h + 2 * g + j) * 16);
    }
    mfmas<NI>(a, b, acc);
  }
}

// A merged step's B code words and scale bytes for a wave, read from LDS a
// step ahead of their use so that the B decode can start right after the
// barrier.  Group g's half of one merged step is 64 elements: A = the merged
// fp16 activation rows, B = weight codes decoded with their block scales;
// the contraction order is the residual step's with the operands swapped
// (lane half h of group g takes elements [32h + 16g, +16) of the step).
template <int NI>
struct MergedB {
  uint2 cb[NI];
  uint32_t sb[NI];
};

template <int NI>
__device__ __forceinline__ void read_merged_b(const uint8_t *st, MergedB<NI> &f, int wn, int g, int lane) {
  using L = Lay<NI>;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = wn * 32 * NI + i * 32 + r;
    f.cb[i] = *reinterpret_cast<const uint2 *>(st + L::XB + row * 32 + slot32(row, h) * 16 + 8 * g);
    f.sb[i] = st[L::XBS + row * 4 + 2 * h + g];
  }
}

// One merged step with the B fragments already read: A rows from LDS, B
// decoded, 2 * NI MFMAs per half.
template <int NI>
__device__ __forceinline__ void mma_merged(const uint8_t *st, const MergedB<NI> &f, f32x16 (&acc)[2][NI], int wm,
                                           int g, int lane) {
  using L = Lay<NI>;
  const int r = lane & 31, h = lane >> 5;
  h2 sb[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) sb[i] = scale_h2(f.sb[i]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint4 a[2], b[NI];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + r;
      a[i] = *reinterpret_cast<const uint4 *>(st + L::XA + row * 128 + slot128(row, 4 * h + 2 * g + j) * 16);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) b[i] = decode8_f16(j ? f.cb[i].y : f.cb[i].x, sb[i]);
    mfmas<NI>(a, b, acc);
  }
}

// One DMA instruction of a thread: source at step 0, bytes per step, LDS
// offset inside a stage, bytes per lane.
struct Dma {
  const uint8_t *g;
  int stride, lds, bytes;
};

}  // namespace dmak

// K % 128 == 0 and (residual) kpad % 64 == 0 (host-checked).  MERGED
// (NI == 2 only): A is the RAC-merged fp16 activation p.x_f16, contracted
// over K alone in 64-element steps; no residual segment.
template <int NI, int EPI, bool HAS_RES, bool MERGED = false>
__global__ __launch_bounds__(dmak::kThreads, NI == 2 ? 4 : 1) void k_gemm_dma(Params p) {
  static_assert(!MERGED || (NI == 2 && !HAS_RES), "merged DMA steps: 128x128 tiles, no residual segment");
  using namespace dmak;
  using L = Lay<NI>;
  using C = typename L::C;
  constexpr int P = L::P;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * L::STAGE];
  __shared__ int s_e, s_m0, s_mend;
  int nt, e, m0, mend;
  if (!tile_setup<C>(p, nt, e, m0, mend, s_e, s_m0, s_mend)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = wave >> 2, wq = wave & 3;
  const int wm = wq / C::WGN, wn = wq % C::WGN;
  auto act_row = [&](int r) -> int64_t {
    int i = m0 + r;
    if (i >= mend) i = mend - 1;  // padding rows re-read a valid row; never stored
    return p.row_token ? static_cast<int64_t>(p.row_token[i]) : static_cast<int64_t>(i);
  };
  auto w_row = [&](int r) -> int64_t { return static_cast<int64_t>(e) * p.N + w_row_of<C, EPI>(r, nt, p.N); };
  const int64_t K = p.K;

  // Wave-instructions of a segment are numbered 0..8P-1; wave w issues its P
  // of them.  Code loads fill 64 16-byte slots per instruction (row = slot/4
  // for 64-byte rows); scale loads fill 64 words (2 per 8-byte row).
  auto code_a = [&](int n) -> Dma {  // activation codes, instruction n (0..7)
    const int pos = 64 * n + lane, row = pos >> 2, c = slot64(row, pos & 3);
    return {p.x_codes + act_row(row) * (K / 2) + c * 16, 64, L::MA + 1024 * n, 16};
  };
  auto code_b = [&](int n) -> Dma {  // weight codes, instruction n (0..BN/16-1)
    const int pos = 64 * n + lane, row = pos >> 2, c = slot64(row, pos & 3);
    return {p.w_codes + w_row(row) * (K / 2) + c * 16, 64, L::MB + 1024 * n, 16};
  };
  auto scale_a = [&](int n) -> Dma {  // activation scales, instruction n (0..3)
    const int pos = 64 * n + lane, row = pos >> 1, half = pos & 1;
    return {p.x_scales + act_row(row) * (K / 16) + half * 4, 8, L::MAS + 256 * n, 4};
  };
  auto scale_b = [&](int n) -> Dma {  // weight scales, instruction n (0..BN/32-1)
    const int pos = 64 * n + lane, row = pos >> 1, half = pos & 1;
    return {p.w_scales + w_row(row) * (K / 16) + half * 4, 8, L::MBS + 256 * n, 4};
  };
  Dma dm[P];
  dm[0] = code_a(wave);
  dm[1] = code_b(wave);
  if constexpr (NI == 2) {
    dm[2] = g == 0 ? scale_a(wq) : scale_b(wq);
  } else {  // 30 loads: waves 6-7 repeat two of the weight-scale loads
    dm[2] = g == 0 ? code_b(8 + wq) : scale_b(wq);
    dm[3] = g == 0 ? scale_a(wq) : scale_b(4 + (wq & 1));
  }
  Dma dr[P];
  if constexpr (HAS_RES) {
    const int64_t kp = p.kpad;
    auto wcols = [&](int n) -> Dma {  // gathered fp16 weight columns, instruction n (0..BN/8-1)
      const int pos = 64 * n + lane, row = pos >> 3, c = slot128(row, pos & 7);
      return {reinterpret_cast<const uint8_t *>(p.wg_f16 + w_row(row) * kp) + c * 16, 128, L::RB + 1024 * n, 16};
    };
#pragma unroll
    for (int q = 0; q < P - 1; ++q) dr[q] = wcols(wave + 8 * q);
    if (g == 0) {  // residual codes, 2 slots per 32-byte row
      const int pos = 64 * wq + lane, row = pos >> 1, c = slot32(row, pos & 1);
      dr[P - 1] = {p.r_codes + act_row(row) * (kp / 2) + c * 16, 32, L::RA + 1024 * wq, 16};
    } else {  // residual scales, 4 bytes per row (waves 6-7 repeat waves 4-5)
      dr[P - 1] = {p.r_scales + act_row(64 * (wq & 1) + lane) * (kp / 16), 4, L::RAS + 256 * (wq & 1), 4};
    }
  }

  f32x16 acc[2][NI];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  if constexpr (MERGED) {
    // Merged fp16 rows: 16 instructions of 8 lanes per 128-byte row; weight
    // codes: 4 of 2 lanes per 32-byte row; weight scales: 2 of 4 bytes per
    // row (waves 6-7 repeat waves 4-5).
    auto xrows = [&](int n) -> Dma {
      const int pos = 64 * n + lane, row = pos >> 3, c = slot128(row, pos & 7);
      return {reinterpret_cast<const uint8_t *>(p.x_f16 + act_row(row) * K) + c * 16, 128, L::XA + 1024 * n, 16};
    };
    Dma dx[P];
#pragma unroll
    for (int q = 0; q < P - 1; ++q) dx[q] = xrows(wave + 8 * q);
    if (g == 0) {
      const int pos = 64 * wq + lane, row = pos >> 1, c = slot32(row, pos & 1);
      dx[P - 1] = {p.w_codes + w_row(row) * (K / 2) + c * 16, 32, L::XB + 1024 * wq, 16};
    } else {
      dx[P - 1] = {p.w_scales + w_row(64 * (wq & 1) + lane) * (K / 16), 4, L::XBS + 256 * (wq & 1), 4};
    }
    const int total = static_cast<int>(K / kStepR);
    auto stage_m = [&](int k) { return lds + (k % kStages) * L::STAGE; };
    auto issue_m = [&](int k) {
      uint8_t *st = stage_m(k);
#pragma unroll
      for (int q = 0; q < P; ++q) dma(dx[q].g + static_cast<int64_t>(k) * dx[q].stride, st + dx[q].lds, dx[q].bytes);
    };
    // Step k+1's B codes and scales are read into registers right after the
    // barrier of step k, so step k+1's decode starts without an LDS wait;
    // step k's A rows are read from its stage.  Step k+2 is issued into the
    // stage of step k-1, whose reads every wave has finished (each waits for
    // its LDS reads before the barrier); step k+1 must have landed by the
    // barrier of step k, one step of DMA look-ahead.
    issue_m(0);
    if (total > 1) issue_m(1);
    if (total > 1) wait_all_but_one_step<P>(); else wait_all();
    barrier_no_fence();
    MergedB<NI> f0, f1;
    read_merged_b<NI>(stage_m(0), f0, wn, g, lane);
    auto step = [&](int k, const MergedB<NI> &cur, MergedB<NI> &next) __attribute__((always_inline)) {
      if (k + 1 < total) {
        wait_all();
        wait_lgkm0();
        barrier_no_fence();
        if (k + 2 < total) issue_m(k + 2);
        read_merged_b<NI>(stage_m(k + 1), next, wn, g, lane);
      }
      mma_merged<NI>(stage_m(k), cur, acc, wm, g, lane);
    };
    for (int k = 0; k < total; k += 2) {
      step(k, f0, f1);
      if (k + 1 < total) step(k + 1, f1, f0);
    }
  } else {
  const int nm = static_cast<int>(K / kStepM);
  const int nr = HAS_RES ? static_cast<int>(p.kpad / kStepR) : 0;
  const int total = nm + nr;
  auto stage = [&](int k) { return lds + (k % kStages) * L::STAGE; };
  auto issue = [&](int k) {
    uint8_t *st = stage(k);
    const Dma *d = k < nm ? dm : dr;
    const int kk = k < nm ? k : k - nm;
#pragma unroll
    for (int q = 0; q < P; ++q) dma(d[q].g + static_cast<int64_t>(kk) * d[q].stride, st + d[q].lds, d[q].bytes);
  };
  issue(0);
  if (total > 1) issue(1);
  for (int k = 0; k < nm; ++k) {
    if (k + 1 < total) wait_all_but_one_step<P>(); else wait_all();
    barrier_no_fence();
    if (k + 2 < total) issue(k + 2);
    compute_main<NI>(stage(k), acc, wm, wn, g, lane);
  }
  if constexpr (HAS_RES) {
    const float ratio = *p.x_g / *p.r_g;  // the residual segment accumulates in units of g_r
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ratio;
    for (int k = nm; k < total; ++k) {
      if (k + 1 < total) wait_all_but_one_step<P>(); else wait_all();
      barrier_no_fence();
      if (k + 2 < total) issue(k + 2);
      compute_res<NI>(stage(k), acc, wm, wn, g, lane);
    }
  }
  }

  // Sum the groups' partial tiles: group 1 hands its accumulators to group 0
  // through LDS, one half (mi) at a time, laid out [wave][ni][r][lane].
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    __syncthreads();
    if (g == 1) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((wq * NI + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] += red[((wq * NI + ni) * 16 + r) * 64 + lane];
    }
  }
  float hmax = 0.0f;
  if (g == 0) hmax = epilogue<C, MERGED ? 2 : 0, EPI, HAS_RES>(p, acc, e, m0, mend, nt, wm, wn, lane);
  if (p.amax_ws != nullptr) amax_gather(p.amax_ws, hmax);  // every thread: it holds a barrier
}

// Exclusive scan of per-expert m-tile counts ceil(rows_e / bm) ->
// tile_offsets[E + 1] by one 256-thread workgroup (E <= 1024: thread t owns
// experts [4t, 4t + 4)).
__device__ void tile_prefix_256(const int32_t *offsets, int E, int bm, int32_t *tile_offsets) {
  __shared__ int32_t wsum[5];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int32_t c[4], own = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    c[q] = e < E ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
    own += c[q];
  }
  int32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (t == 0) {
    int32_t run = 0;
    for (int w = 0; w < 4; ++w) {
      const int32_t x = wsum[w];
      wsum[w] = run;
      run += x;
    }
    wsum[4] = run;
  }
  __syncthreads();
  int32_t run = wsum[wave] + incl - own;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e < E) tile_offsets[e] = run;
    run += c[q];
  }
  if (t == 0) tile_offsets[E] = wsum[4];
}

__global__ __launch_bounds__(256) void k_tile_prefix(const int32_t *offsets, int E, int bm, int32_t *tile_offsets) {
  tile_prefix_256(offsets, E, bm, tile_offsets);
}

// Gather the selected weight columns of every expert row into fp16
// [E*N, kpad] (exact values e2m1 * e4m3, no tensor scale).  One row per
// 64-thread quarter of the workgroup: the row's codes and scales are staged in
// LDS, then each thread emits 8 consecutive outputs (one 16-byte store).
// The launch has one workgroup more than the gather needs; the last one
// builds the per-expert tile prefix instead (one launch for both).
__global__ __launch_bounds__(256) void k_gather_wcols(const uint8_t *w_codes, const uint8_t *w_scales,
                                                      int64_t rows_total, int K, const int32_t *sel,
                                                      int kpad, uint16_t *out, const int32_t *offsets, int E,
                                                      int bm, int32_t *tile_offsets) {
  extern __shared__ uint4 gather_lds[];
  if (blockIdx.x == gridDim.x - 1) {
    tile_prefix_256(offsets, E, bm, tile_offsets);
    return;
  }
  const int q = threadIdx.x >> 6, t = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + q;
  const int stride = (K / 2 + K / 16 + 15) / 16 * 16;
  uint8_t *mine = reinterpret_cast<uint8_t *>(gather_lds) + q * stride;
  if (row < rows_total) {
    const uint2 *c = reinterpret_cast<const uint2 *>(w_codes + row * (K / 2));
    for (int i = t; i < K / 16; i += 64) reinterpret_cast<uint2 *>(mine)[i] = c[i];
    const uint8_t *s = w_scales + row * (K / 16);
    for (int i = t; i < K / 16; i += 64) mine[K / 2 + i] = s[i];
  }
  __syncthreads();
  if (row >= rows_total) return;
  for (int g = t; g < kpad / 8; g += 64) {
    const int4 i0 = reinterpret_cast<const int4 *>(sel)[2 * g];
    const int4 i1 = reinterpret_cast<const int4 *>(sel)[2 * g + 1];
    const int idx[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = idx[k];
      const uint32_t code = (mine[c >> 1] >> ((c & 1) * 4)) & 0xFu;
      const float v = dequant_code(code, e4m3_to_f32(mine[K / 2 + (c >> 4)]));
      h[k] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
    reinterpret_cast<uint4 *>(out + row * kpad)[g] =
        make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  }
}

using CfgS = Cfg<128, 128, 2, 2, 2>;  // general / ragged shapes: 256 threads, 2 workgroups per CU
using CfgL = Cfg<256, 256, 2, 4, 1>;  // large grouped shapes: 512 threads, 128x64 wave tiles

// kS: register-staged 128x128; kL: register-staged 256x256 (NVFP4 operands);
// kP: ping-pong 256x256 (bf16 operands); kD: DMA-staged 128x128 (NVFP4).
enum TileCfg { kS = 0, kL = 2, kP = 4, kD = 7 };

// The DMA-staged kernel's shape limits: NVFP4 operands, 128-element main
// steps, 64-element residual steps.
bool dma_fits(const GemmLaunch &a) {
  const bool res = a.r_codes != nullptr && a.kpad > 0;
  return a.mode == 0 && a.K % 128 == 0 && a.N % 128 == 0 && (!res || a.kpad % 64 == 0);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Pick the tile shape from host-known sizes only (per-expert row counts live
// on the device): estimated CU occupancy x expected per-workgroup efficiency
// x fraction of tile rows that are real rows.
TileCfg pick_cfg(const GemmLaunch &a) {
  struct Cand {
    TileCfg c;
    int bm, bn, slots;
    double eff;
  } cands[2] = {{kS, 128, 128, 512, 0.6}, {kL, 256, 256, 256, 1.0}};
  TileCfg best = kS;
  double best_score = -1.0;
  // Large tiles: the ping-pong kernel wins for bf16 operands, the plain
  // 8-wave kernel for NVFP4 operands (whose decode already overlaps the MFMAs).
  const TileCfg large = a.mode != 0 ? kP : kL;
  for (const Cand &c : cands) {
    if (a.N % c.bn) continue;
    const double m_est = static_cast<double>((a.num_rows + c.bm - 1) / c.bm) + (a.E > 1 ? a.E / 2.0 : 0.0);
    const double wgs = m_est * static_cast<double>(a.N / c.bn);
    const double rounds = wgs > 0 ? static_cast<double>(static_cast<int64_t>((wgs + c.slots - 1) / c.slots)) : 1.0;
    const double util = wgs / (rounds * c.slots);
    const double pad = m_est > 0 ? static_cast<double>(a.num_rows) / (m_est * c.bm) : 0.0;
    const double score = util * c.eff * (pad > 1.0 ? 1.0 : pad);
    if (score > best_score) {
      best_score = score;
      best = c.c == kL ? large : c.c;
    }
  }
  // 128x128 NVFP4 tiles: the DMA-staged kernel where its shape limits allow
  // (measured 61 vs 70 us on 4096x1536x(2048+1024)); the large-tile kernel
  // stays ahead on many-tile grouped shapes.
  if (best == kS && dma_fits(a)) best = kD;
  return best;
}

int cfg_bm(TileCfg c) { return (c == kL || c == kP) ? 256 : 128; }
int cfg_bn(TileCfg c) { return (c == kL || c == kP) ? 256 : CfgS::BN; }

template <class C, int MODE, int EPI, bool RES>
void launch_k(const Params &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm<C, MODE, EPI, RES>), dim3(grid), dim3(C::THREADS), 0, s, p);
}

template <int MODE, int EPI, bool RES>
void launch_pp(const Params &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_pp<MODE, EPI, RES>), dim3(grid), dim3(CfgPP::THREADS), 0, s, p);
}

void launch_pp_cfg(const GemmLaunch &a, const Params &p, int g, bool res, hipStream_t stream) {
  if (a.mode == 1) {
    if (a.epilogue == 0) launch_pp<1, 0, false>(p, g, stream);
    else launch_pp<1, 1, false>(p, g, stream);
  } else if (a.mode == 2) {
    if (a.epilogue == 0) launch_pp<3, 0, false>(p, g, stream);
    else launch_pp<3, 1, false>(p, g, stream);
  } else if (a.mode == 3) {
    if (a.epilogue == 0) launch_pp<4, 0, false>(p, g, stream);
    else launch_pp<4, 1, false>(p, g, stream);
  } else if (res) {
    if (a.epilogue == 0) launch_pp<0, 0, true>(p, g, stream);
    else launch_pp<0, 1, true>(p, g, stream);
  } else {
    if (a.epilogue == 0) launch_pp<0, 0, false>(p, g, stream);
    else launch_pp<0, 1, false>(p, g, stream);
  }
}

template <int NI>
void launch_dma(const GemmLaunch &a, const Params &p, int g, bool res, hipStream_t s, bool merged = false) {
  const dim3 grid(g), block(dmak::kThreads);
  if constexpr (NI == 2) {
    if (merged) {
      if (a.epilogue == 0) hipLaunchKernelGGL((k_gemm_dma<2, 0, false, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_gemm_dma<2, 1, false, true>), grid, block, 0, s, p);
      return;
    }
  }
  if (res) {
    if (a.epilogue == 0) hipLaunchKernelGGL((k_gemm_dma<NI, 0, true>), grid, block, 0, s, p);
    else if constexpr (NI % 2 == 0) hipLaunchKernelGGL((k_gemm_dma<NI, 1, true>), grid, block, 0, s, p);
  } else {
    if (a.epilogue == 0) hipLaunchKernelGGL((k_gemm_dma<NI, 0, false>), grid, block, 0, s, p);
    else if constexpr (NI % 2 == 0) hipLaunchKernelGGL((k_gemm_dma<NI, 1, false>), grid, block, 0, s, p);
  }
}

template <class C>
void launch_cfg(const GemmLaunch &a, const Params &p, int g, bool res, hipStream_t stream, bool merged = false) {
  if (merged) {
    if (a.epilogue == 0) launch_k<C, 2, 0, false>(p, g, stream);
    else if constexpr (C::NI % 2 == 0) launch_k<C, 2, 1, false>(p, g, stream);
  } else if (a.mode != 0) {
    // bf16 operands: large tiles run on the ping-pong kernel (pick_cfg), so
    // only the 128 x 128 register-staged kernel is instantiated for them
    if constexpr (C::BM == 128) {
      if (a.mode == 1) {
        if (a.epilogue == 0) launch_k<C, 1, 0, false>(p, g, stream);
        else launch_k<C, 1, 1, false>(p, g, stream);
      } else if (a.mode == 2) {
        if (a.epilogue == 0) launch_k<C, 3, 0, false>(p, g, stream);
        else launch_k<C, 3, 1, false>(p, g, stream);
      } else {
        if (a.epilogue == 0) launch_k<C, 4, 0, false>(p, g, stream);
        else launch_k<C, 4, 1, false>(p, g, stream);
      }
    }
  } else if (res) {
    if (a.epilogue == 0) launch_k<C, 0, 0, true>(p, g, stream);
    else if constexpr (C::NI % 2 == 0) launch_k<C, 0, 1, true>(p, g, stream);
  } else {
    if (a.epilogue == 0) launch_k<C, 0, 0, false>(p, g, stream);
    else if constexpr (C::NI % 2 == 0) launch_k<C, 0, 1, false>(p, g, stream);
  }
}

// RAC calls with many rows per expert: which formulation of the correction.
// QUADS_RAC_FORM_EXACT and _MERGED choose it; QUADS_RAC_FORM_AUTO takes the
// merged fp16 activation operand (MODE 2: one MFMA pass over K, after a merge
// pass) where the extended-K GEMM would run on the large register-staged
// tiles (measured on the 16384-token prefill layer: 0.94 vs 1.30 ms gate_up,
// 0.64 vs 0.83 ms down, merge passes included); on the 128x128 DMA-staged
// shapes the merge pass costs what the shorter GEMM saves (4096 x 1536 x
// 2048: 18 + 48 vs 5 + 62 us), so the exact extended-K kernel stays.  A
// merged operand the caller built (quads_rac_select_merged) is always taken:
// the DMA-staged 128x128 kernel reads it as well.
bool use_merged(const GemmLaunch &a) {
  if (a.mode != 0 || a.r_codes == nullptr || a.kpad == 0 || gemm_use_small(a)) return false;
  if (a.x_merged != nullptr || a.rac_form == QUADS_RAC_FORM_MERGED) return true;
  if (a.rac_form == QUADS_RAC_FORM_EXACT || rac_rows_per_group(a.K, a.kpad, true) < 1) return false;
  const TileCfg c = pick_cfg(a);
  return c == kL || c == kP;
}

// The register-staged NVFP4 kernels address the activation tensor and one
// expert's weights through buffer resources: 32-bit byte offsets.
bool buf_fits(const GemmLaunch &a, bool merged) {
  constexpr int64_t kMax = int64_t(1) << 32;
  const int64_t act = merged ? a.act_rows * a.K * 2 : a.act_rows * (a.K / 2);
  return act < kMax && a.N * (a.K / 2) < kMax;
}

TileCfg pick_cfg_for(const GemmLaunch &a) {
  TileCfg c = pick_cfg(a);
  const bool merged = use_merged(a);
  if (merged && c == kP) c = kL;  // kD, kS and kL have a merged form
  // The merged fp16 operand on 128x128 tiles: the register-staged kernel
  // (4096 x 1536 x 2048 step 73 against 78 us); NVFP4 activation codes and
  // the extended-K form stay on the DMA-staged kernel (51 against 53 us,
  // 91 against 93.5 us).
  if (merged && c == kD) c = kS;
  if (a.mode == 0 && (c == kL || c == kS) && !buf_fits(a, merged)) c = kD;  // dma_fits (gemm_shape_supported)
  return c;
}

}  // namespace

namespace {
size_t gemm_ws_base(const GemmLaunch &a) {
  size_t b = align256(static_cast<size_t>(a.E + 1) * sizeof(int32_t));
  if (a.mode == 0 && a.r_codes != nullptr && a.kpad > 0 && a.x_merged == nullptr)
    b += (gemm_use_small(a) || use_merged(a)) ? align256(gemm_small_res_bytes(a))
                                              : align256(static_cast<size_t>(a.E) * a.N * a.kpad * sizeof(uint16_t));
  return b;
}

// The amax word is only touched with system-scope atomics (where the
// gathering atomic maxima from every XCD are performed).
__global__ __launch_bounds__(64) void k_zero_words(uint32_t *p, int n) {
  if (static_cast<int>(threadIdx.x) < n) __hip_atomic_store(p + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The output's tensor scale from the amax the GEMM gathered (the fold the
// quantizer applies to its own amax), and the words cleared for the next call.
__global__ __launch_bounds__(64) void k_fold_amax(uint32_t *words, float *gscale) {
  static_assert(kAmaxWords == 64, "one word per lane");
  const uint32_t m = __hip_atomic_exchange(words + threadIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const uint32_t t = last_lane(wave_scan<true>(m));
  if (threadIdx.x == 0) *gscale = tensor_scale_from_amax(__uint_as_float(t));
}
}  // namespace

bool gemm_shape_supported(const GemmLaunch &a) {
  return a.mode != 0 || gemm_use_small(a) || buf_fits(a, use_merged(a)) || dma_fits(a);
}

size_t gemm_ws_bytes(const GemmLaunch &a) {
  return gemm_ws_base(a) + (a.y_gscale != nullptr ? kAmaxWords * sizeof(uint32_t) : 0);
}

hipError_t launch_fold_amax(const GemmLaunch &a, hipStream_t stream) {
  if (a.y_gscale == nullptr) return hipSuccess;
  hipLaunchKernelGGL(k_fold_amax, dim3(1), dim3(64), 0, stream, gemm_amax_words(a), a.y_gscale);
  return hipGetLastError();
}

uint32_t *gemm_amax_words(const GemmLaunch &a) {
  if (a.y_gscale == nullptr) return nullptr;
  return reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(a.ws) + gemm_ws_base(a));
}

hipError_t launch_gemm_prepare(const GemmLaunch &a, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  int32_t *tile_offsets = reinterpret_cast<int32_t *>(ws);
  if (uint32_t *words = gemm_amax_words(a)) {  // the main kernel's amax word starts at zero
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, stream, words, kAmaxWords);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool res = a.mode == 0 && a.r_codes != nullptr && a.kpad > 0;
  if (gemm_use_small(a)) {
    uint16_t *rd = reinterpret_cast<uint16_t *>(ws + align256((a.E + 1) * sizeof(int32_t)));
    return res && a.x_merged == nullptr ? launch_gemm_small_prepare(a, rd, stream) : hipSuccess;
  }
  const TileCfg c = pick_cfg_for(a);
  if (use_merged(a)) {
    if (a.x_merged == nullptr) {
      uint16_t *xm = reinterpret_cast<uint16_t *>(ws + align256((a.E + 1) * sizeof(int32_t)));
      const hipError_t e = launch_gemm_small_prepare(a, xm, stream);
      if (e != hipSuccess) return e;
    }
    if (a.E > 1)
      hipLaunchKernelGGL(k_tile_prefix, dim3(1), dim3(256), 0, stream, a.expert_offsets, a.E, cfg_bm(c),
                         tile_offsets);
  } else if (res) {
    uint16_t *wg = reinterpret_cast<uint16_t *>(ws + align256((a.E + 1) * sizeof(int32_t)));
    const int64_t rows_total = static_cast<int64_t>(a.E) * a.N;
    const int K = static_cast<int>(a.K);
    const size_t lds = 4 * ((K / 2 + K / 16 + 15) / 16 * 16);
    hipLaunchKernelGGL(k_gather_wcols, dim3((rows_total + 3) / 4 + 1), dim3(256), lds, stream, a.w_codes,
                       a.w_scales, rows_total, K, a.sel_idx, static_cast<int>(a.kpad), wg, a.expert_offsets, a.E,
                       cfg_bm(c), tile_offsets);
  } else if (a.E > 1) {  // one expert: the kernels read its tiles off expert_offsets
    hipLaunchKernelGGL(k_tile_prefix, dim3(1), dim3(256), 0, stream, a.expert_offsets, a.E, cfg_bm(c), tile_offsets);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_main(const GemmLaunch &a, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  int32_t *tile_offsets = reinterpret_cast<int32_t *>(ws);
  const bool res = a.mode == 0 && a.r_codes != nullptr && a.kpad > 0;
  uint16_t *wg = res ? reinterpret_cast<uint16_t *>(ws + align256((a.E + 1) * sizeof(int32_t))) : nullptr;
  if (res && a.x_merged != nullptr) wg = const_cast<uint16_t *>(a.x_merged);  // read only
  if (gemm_use_small(a)) return launch_gemm_small(a, wg, stream);
  const bool merged = use_merged(a);
  const TileCfg c = pick_cfg_for(a);
  const int bm = cfg_bm(c), bn = cfg_bn(c);
  Params p{};
  p.expert_offsets = a.expert_offsets;
  p.tile_offsets = tile_offsets;
  p.E = a.E;
  p.n_seg = a.n_seg;
  p.N = a.N;
  p.K = a.K;
  p.kpad = a.kpad;
  p.act_rows = a.act_rows;
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
  p.wg_f16 = merged ? nullptr : wg;
  p.x_f16 = merged ? wg : nullptr;
  p.y = a.y;
  p.y_bf16 = a.y_bf16 ? 1 : 0;
  p.amax_ws = gemm_amax_words(a);
  p.n_tiles = static_cast<int>(a.N / bn);
  const int64_t m_tiles = (a.num_rows + bm - 1) / bm + a.E;
  int64_t grid = m_tiles * p.n_tiles;
  grid = (grid + 7) / 8 * 8;
  const int g = static_cast<int>(grid);
  if (c == kD) launch_dma<2>(a, p, g, res, stream, merged);
  else if (c == kP) launch_pp_cfg(a, p, g, res, stream);
  else if (c == kL) launch_cfg<CfgL>(a, p, g, res, stream, merged);
  else launch_cfg<CfgS>(a, p, g, res, stream, merged);
  return hipGetLastError();
}

}  // namespace quads
