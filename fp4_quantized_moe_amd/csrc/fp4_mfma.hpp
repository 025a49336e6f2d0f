// NVFP4 -> fp16 operand decode for the fp16 MFMA GEMM kernels (gfx950).
//
// An NVFP4 value e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16; fp16 products are exact in FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quads {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// (dec(s), dec(s)) as fp16 for an E4M3 scale byte s: exact conversion.
__device__ __forceinline__ h2 scale_h2(uint32_t s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s | (s << 8), 1.0f, false);
}

// 8 E2M1 codes (element i in nibble i) times the block scale -> 8 fp16.
__device__ __forceinline__ uint4 decode8_f16(uint32_t w, h2 sc) {
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

}  // namespace quads
