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

// One 16-element block quantized: packed codes (element i in nibble i of the
// 64-bit word lo | hi << 32) and the E4M3 scale byte.
struct BlockQ {
  uint32_t lo, hi;  // codes of elements 0..7 and 8..15
  uint32_t scale;
};

// RN(a / d) for finite a >= 0 and normal d > 0, given r = RN(1 / d):
// q = RN(a r) is within one ulp of a/d, the remainder a - d q is exact in one
// FMA, and RN(q + (a - d q) r) is the correctly rounded quotient (Markstein's
// theorem for round-to-nearest).  Quotients small enough to underflow are far
// below the first E2M1 rounding threshold (0.25), so they cannot change a code.
__device__ __forceinline__ float div_rn_with_rcp(float a, float d, float r) {
  const float q = a * r;
  const float e = __builtin_fmaf(-d, q, a);
  return __builtin_fmaf(e, r, q);
}

// Quantize 16 values with tensor scale g.  The E2M1 rounding (nearest, ties
// to even, saturating at 6, sign kept for zeros) and the nibble packing are
// done by v_cvt_scalef32_pk_fp4_f32 with a unit scale on the exact quotient
// fl32(x / d); its rounding equals the threshold rule of e2m1_index on every
// FP32 input (checked exhaustively over the rounding-relevant range).  If
// `dq_out` is non-null, writes dq = sign * fl32(level * d), decoding the codes
// back with v_cvt_scalef32_pk_f32_fp4.
__device__ __forceinline__ BlockQ quantize_block16(const float (&x)[16], float g, float *dq_out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float s_real = (amax / 6.0f) / g;
  const uint32_t s = f32_to_e4m3(s_real);
  const float d = e4m3_to_f32(s) * g;
  float v[16];
  if (d >= 0x1p-125f) {
    const float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_copysignf(div_rn_with_rcp(fabsf(x[i]), d, r), x[i]);
  } else if (d > 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x[i] / d;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_copysignf(0.0f, x[i]);
  }
  BlockQ q;
  q.scale = s;
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[0], v[1], 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2], v[3], 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[4], v[5], 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[6], v[7], 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[8], v[9], 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[10], v[11], 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[12], v[13], 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[14], v[15], 1.0f, 3);
  q.lo = lo;
  q.hi = hi;
  if (dq_out) {
#define QUADS_DQ_BYTE(word, byte, base)                                            \
  {                                                                                \
    const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, byte);     \
    dq_out[(base)] = e[0] * d;                                                     \
    dq_out[(base) + 1] = e[1] * d;                                                 \
  }
    QUADS_DQ_BYTE(lo, 0, 0)
    QUADS_DQ_BYTE(lo, 1, 2)
    QUADS_DQ_BYTE(lo, 2, 4)
    QUADS_DQ_BYTE(lo, 3, 6)
    QUADS_DQ_BYTE(hi, 0, 8)
    QUADS_DQ_BYTE(hi, 1, 10)
    QUADS_DQ_BYTE(hi, 2, 12)
    QUADS_DQ_BYTE(hi, 3, 14)
#undef QUADS_DQ_BYTE
  }
  return q;
}

// Dequantized FP32 value of one code given the block's d = fl32(dec(s) * g).
__device__ __forceinline__ float dequant_code(uint32_t code, float d) {
  const float m = e2m1_level(code & 7u) * d;
  return (code & 8u) ? -m : m;
}

}  // namespace quads
