// Device-side NVFP4 codec and small helpers for the gfx950 kernels.
//
// NVFP4 as this library encodes it: E2M1 elements (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6 -- the eight levels per sign the QUADS technical summary,
// section 1, refers to), one OCP E4M3 scale per 16 elements, one FP32 scale
// per tensor.  All roundings are nearest-even with saturation.  Every FP32
// step below is a single IEEE operation: the library is built with
// -ffp-contract=off, IEEE-correct division and FP32 denormals preserved, so
// the codes, scales and residuals match a plain FP32 evaluation bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quads {

constexpr float kTensorScaleDivisor = 2688.0f;  // 6 (E2M1 max) * 448 (E4M3 max)

// E4M3 byte (0x00..0x7E) -> exact FP32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t s) {
  const uint32_t e = (s >> 3) & 0xFu, m = s & 7u;
  if (e == 0) return static_cast<float>(m) * 0x1p-9f;  // subnormal: m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Finite v >= 0 -> E4M3 byte, nearest-even, saturating to 448 (0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0x1p-6f) {
    // Subnormal range: step 2^-9.  v * 512 is exact; rint is nearest-even.
    // A result of 8 is 2^-6, which is exactly code 0x08 (the first normal).
    return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));
  }
  uint32_t b = __float_as_uint(v);
  b = b + 0x7FFFFu + ((b >> 20) & 1u);  // keep 3 mantissa bits, ties to even
  return (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

// Nearest E2M1 magnitude index (0..7) of v >= 0, ties to the even index,
// saturating at 6.  The comparisons are the midpoints of adjacent levels;
// "<=" where the lower neighbour has the even index, "<" where the upper does.
__device__ __forceinline__ uint32_t e2m1_index(float v) {
  return static_cast<uint32_t>(v > 0.25f) + static_cast<uint32_t>(v >= 0.75f) +
         static_cast<uint32_t>(v > 1.25f) + static_cast<uint32_t>(v >= 1.75f) +
         static_cast<uint32_t>(v > 2.5f) + static_cast<uint32_t>(v >= 3.5f) +
         static_cast<uint32_t>(v > 5.0f);
}

// E2M1 magnitude index -> FP32 level, built from its bits:
// index 1 is 0.5; index i >= 2 is 2^((i>>1)-1) * (1 + (i&1)/2).
__device__ __forceinline__ float e2m1_level(uint32_t i) {
  const uint32_t normal = ((((i >> 1) + 126u) << 23) | ((i & 1u) << 22));
  const uint32_t bits = i >= 2u ? normal : (i == 1u ? 0x3F000000u : 0u);
  return __uint_as_float(bits);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Per-tensor scale from the tensor's amax.
__device__ __forceinline__ float tensor_scale_from_amax(float a) {
  return a == 0.0f ? 1.0f : a / kTensorScaleDivisor;
}

// FP32 -> bf16 bits, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// silu(z) = z / (1 + e^-z) in FP32 for the SwiGLU epilogues: e^-z as
// 2^(-z log2 e) (v_exp_f32) and the quotient as z times the hardware
// reciprocal (v_rcp_f32), a few ulp of FP32 against the bf16 rounding (2^-9)
// of the stored product.  Large |z| give the limits: z >> 0 -> z, z << 0 -> -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// One 16-element block quantized: packed codes (element i in nibble i of the
// 64-bit word lo | hi << 32) and the E4M3 scale byte.
struct BlockQ {
  uint32_t lo, hi;  // codes of elements 0..7 and 8..15
  uint32_t scale;
};

// RN(a / d) for finite a >= 0 and d in [2^-125, 2^126), given r = RN(1 / d):
// q = RN(a r) is within one ulp of a/d, the remainder a - d q is exact in one
// FMA, and RN(q + (a - d q) r) is the correctly rounded quotient (Markstein's
// theorem for round-to-nearest).  Quotients small enough to underflow are far
// below the first E2M1 rounding threshold (0.25), so they cannot change a code.
__device__ __forceinline__ float div_rn_with_rcp(float a, float d, float r) {
  const float q = a * r;
  const float e = __builtin_fmaf(-d, q, a);
  return __builtin_fmaf(e, r, q);
}

// A tensor scale g with its rounded reciprocal, for the block-scale division
// fl32(a / g).  `fast` holds where the reciprocal-corrected division is the
// correctly rounded quotient (g and 1/g normal).
struct TensorScale {
  float g, rg;
  bool fast;
};

__device__ __forceinline__ TensorScale tensor_scale(float g) {
  return {g, 1.0f / g, g >= 0x1p-125f && g < 0x1p126f};
}

// Block scale of a 16-element block with amax `amax` under tensor scale g:
// s = E4M3(fl32(fl32(amax / 6) / g)) and d = fl32(dec(s) * g).  Both
// divisions are the correctly rounded quotients: fl32(amax / 6) by the
// reciprocal-corrected division with RN(1/6) while the quotient is a normal
// number (amax >= 2^-100), and fl32(a / g) by the same with RN(1/g), the
// dividend capped at 1024 g (quotients above 448 saturate the scale whatever
// their value, and the cap keeps the corrected division from overflowing);
// other operands take a plain division.
struct BlockScale {
  uint32_t s;
  float d;
};

__device__ __forceinline__ BlockScale block_scale(float amax, const TensorScale &ts) {
  constexpr float kRcp6 = 0x1.555556p-3f;  // RN(1/6)
  float s6, s_real;
  if (__builtin_expect(amax >= 0x1p-100f, 1)) s6 = div_rn_with_rcp(amax, 6.0f, kRcp6);
  else s6 = amax / 6.0f;
  if (__builtin_expect(ts.fast, 1)) s_real = div_rn_with_rcp(fminf(s6, 1024.0f * ts.g), ts.g, ts.rg);
  else s_real = s6 / ts.g;
  const uint32_t s = f32_to_e4m3(s_real);
  return {s, e4m3_to_f32(s) * ts.g};
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed bf16 (a in the low half), nearest-even, with
// gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Signed quotients of N elements of one block, branch-free, that round to
// the same E2M1 codes as the exact v[i] = fl32(x[i] / d):
//   - d outside [2^-125, 2^126) is first brought into that range by an exact
//     power-of-two scaling of both operands (2^64 up or down), which leaves
//     the quotient's real value unchanged, so the reciprocal-corrected
//     division below is the correctly rounded quotient (and dividends that
//     lose bits when scaled down have quotients far below the first rounding
//     threshold, 0.25);
//   - the dividend is capped at 8 d: every quotient above 5 takes the top
//     level (6) whatever its value, and the cap keeps the corrected division
//     from overflowing (possible when a given tensor scale is far too small
//     for the data);
//   - d == 0 gives zero with the sign of x.
// Blocks with d in the normal range (all but degenerate tensors) take the
// short form: cap, corrected division, sign.
template <int N>
__device__ __forceinline__ void block_quotients(const float (&x)[N], float d, float (&v)[N]) {
  if (__builtin_expect(d >= 0x1p-125f && d < 0x1p126f, 1)) {
    const float r = 1.0f / d;
    const float cap = 8.0f * d;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __builtin_copysignf(div_rn_with_rcp(fminf(fabsf(x[i]), cap), d, r), x[i]);
  } else {
    const float sc = d < 0x1p-125f ? 0x1p64f : 0x1p-64f;
    const float dd = d * sc;
    const float r = 1.0f / dd;
    const float cap = 8.0f * dd;
    const bool live = d > 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float a = fminf(fabsf(x[i]) * sc, cap);
      v[i] = __builtin_copysignf(live ? div_rn_with_rcp(a, dd, r) : 0.0f, x[i]);
    }
  }
}

// E2M1 codes of 8 quotients (element i in nibble i): nearest, ties to even,
// saturating at 6, sign kept for zeros.  v_cvt_scalef32_pk_fp4_f32 with a
// unit scale rounds exactly as the threshold rule of e2m1_index on every
// FP32 input (checked exhaustively over the rounding-relevant range).
__device__ __forceinline__ uint32_t pack8_fp4(const float *v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// dq = sign * fl32(level * d) of the 8 codes of a word, decoded with
// v_cvt_scalef32_pk_f32_fp4 (unit scale: the exact signed level).
template <int B>
__device__ __forceinline__ void dequant_byte(uint32_t w, float d, float *dq) {
  const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  dq[2 * B] = e[0] * d;
  dq[2 * B + 1] = e[1] * d;
}

__device__ __forceinline__ void dequant8(uint32_t w, float d, float *dq) {
  dequant_byte<0>(w, d, dq);
  dequant_byte<1>(w, d, dq);
  dequant_byte<2>(w, d, dq);
  dequant_byte<3>(w, d, dq);
}

// The 16 values of a block's codes (codes.x: elements 0-7, codes.y: 8-15)
// times d >= 0, exact in FP32, with the code's sign also on zeros: the
// negative-zero code gives -0 (the hardware conversion alone gives +0).
template <int B>
__device__ __forceinline__ void dequant_byte_signed(uint32_t w, float d, float *v) {
  const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t sign = (w << (28 - 4 * (2 * B + u))) & 0x80000000u;  // bit 3 of nibble 2B+u
    v[2 * B + u] = __uint_as_float(__float_as_uint(e[u] * d) | sign);
  }
}

__device__ __forceinline__ void dequant16_signed(uint2 codes, float d, float (&v)[16]) {
  dequant_byte_signed<0>(codes.x, d, v);
  dequant_byte_signed<1>(codes.x, d, v);
  dequant_byte_signed<2>(codes.x, d, v);
  dequant_byte_signed<3>(codes.x, d, v);
  dequant_byte_signed<0>(codes.y, d, v + 8);
  dequant_byte_signed<1>(codes.y, d, v + 8);
  dequant_byte_signed<2>(codes.y, d, v + 8);
  dequant_byte_signed<3>(codes.y, d, v + 8);
}

// One 16-element block of the RAC-merged fp16 operand (units of the
// activation's tensor scale g_x): element i is X'_i, or, where bit i of
// `sel` is set, fl32(X'_i + cor_i) with cor_i = fl32(R' * fl32(g_r / g_x))
// its channel's correction; then one rounding to fp16 (RNE).  X' and R' are
// the exact e2m1 * e4m3 values.  Element 0 lands in the low half of lo.x.
__device__ __forceinline__ void merged_block16(const float (&xv)[16], const float (&cor)[16], uint32_t sel,
                                               uint4 &lo, uint4 &hi) {
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * i + u;
      const float s = xv[e] + cor[e];
      v[u] = (sel >> e) & 1u ? s : xv[e];
    }
    h[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[0]))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[1]))) << 16);
  }
  lo = make_uint4(h[0], h[1], h[2], h[3]);
  hi = make_uint4(h[4], h[5], h[6], h[7]);
}

// Quantize 16 values with tensor scale g: the block scale from their amax,
// the quotients fl32(x / d), their E2M1 codes, and (if `dq_out` is non-null)
// the dequantized values.
__device__ __forceinline__ BlockQ quantize_block16(const float (&x)[16], const TensorScale &ts, float *dq_out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const BlockScale bs = block_scale(amax, ts);
  float v[16];
  block_quotients<16>(x, bs.d, v);
  BlockQ q;
  q.scale = bs.s;
  q.lo = pack8_fp4(v);
  q.hi = pack8_fp4(v + 8);
  if (dq_out) {
    dequant8(q.lo, bs.d, dq_out);
    dequant8(q.hi, bs.d, dq_out + 8);
  }
  return q;
}

// Fake-quantized (QDQ) bf16 values of one half (8 consecutive elements) of a
// 16-element block, given the whole block's amax: bf16_RNE(dq) with the same
// operations quantize_block16 applies to each element, so the bits equal the
// quantizer's QDQ output for that block.  Returns the 8 bf16 values packed
// two per word, element 0 in the low half of word 0.
__device__ __forceinline__ uint4 qdq8_bf16(const float (&x)[8], float amax, const TensorScale &ts) {
  const BlockScale bs = block_scale(amax, ts);
  float v[8];
  block_quotients<8>(x, bs.d, v);
  float dq[8];
  dequant8(pack8_fp4(v), bs.d, dq);
  return make_uint4(pack_bf16x2(dq[0], dq[1]), pack_bf16x2(dq[2], dq[3]), pack_bf16x2(dq[4], dq[5]),
                    pack_bf16x2(dq[6], dq[7]));
}

// Wave-wide inclusive scans with DPP moves (no LDS round trip): shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane of row r
// is added to row r + 1 (row_bcast:15) and lane 31 to rows 2 and 3
// (row_bcast:31).  Lanes whose source is outside the row keep 0, the
// identity of both operations here (unsigned sum and max).
template <bool MAX>
__device__ __forceinline__ uint32_t dpp_op(uint32_t a, uint32_t b) {
  return MAX ? (a > b ? a : b) : a + b;
}

template <bool MAX>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = dpp_op<MAX>(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return v;
}

// The value of lane 63 (after a scan: the wave total), as a uniform value.
__device__ __forceinline__ uint32_t last_lane(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// The amax of a kernel's bf16 output, gathered while the kernel writes it:
// each thread passes the largest |value| it stored (fmaxf of the stored bf16
// values, so NaN is skipped as the quantizer's amax skips it); the workgroup
// reduces them (non-negative floats order like their bit patterns) and one
// atomic max per workgroup lands in words[blockIdx.x % kAmaxWords], spread
// so that few atomics meet at one address.  System scope, so that maxima
// from every XCD meet in one place; no value is awaited.  The words must be
// zero before the launch; a later launch folds them (k_fold_amax).  Contains
// a barrier: every thread of the workgroup calls it.
constexpr int kAmaxWords = 64;

// `red`: 16 words of LDS the caller is done with (every thread calls).
__device__ __forceinline__ void amax_gather(uint32_t *words, float m, uint32_t *red) {
  const uint32_t wm = last_lane(wave_scan<true>(__float_as_uint(m)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < static_cast<int>((blockDim.x + 63) >> 6); ++w) t = max(t, red[w]);
    if (t != 0u)
      __hip_atomic_fetch_max(words + blockIdx.x % kAmaxWords, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__device__ __forceinline__ void amax_gather(uint32_t *words, float m) {
  __shared__ uint32_t red[16];
  amax_gather(words, m, red);
}

// Dequantized FP32 value of one code given the block's d = fl32(dec(s) * g).
__device__ __forceinline__ float dequant_code(uint32_t code, float d) {
  const float m = e2m1_level(code & 7u) * d;
  return (code & 8u) ? -m : m;
}

}  // namespace quads
