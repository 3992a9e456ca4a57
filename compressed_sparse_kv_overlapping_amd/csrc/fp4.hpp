// MX decoding on gfx950: MXFP4 (shared by the indexer and the attention
// kernels) and MXFP8 with E4M3 elements (attention entries).
//
// MXFP4 (OCP Microscaling v1.0): 32 FP4 E2M1 elements share one E8M0 scale
// 2^(X-127).  Rows are stored as code bytes, element 2j in the low nibble of
// byte j, plus a separate array of scale bytes, one per 32 elements.  An
// E2M1 value times a power of two has at most two significant bits, so the
// decode to bf16 is exact while the value lies in bf16's (= fp32's) normal
// range.
#pragma once
#include "common.hpp"

namespace cskv {

// E8M0 scale X as the fp32 2^(X-127): X = 0 is the subnormal 2^-127 and
// X = 255 (NaN in E8M0) a NaN, so that the value is right whether the
// conversion reads the whole fp32 or only its exponent field.
__device__ __forceinline__ uint32_t e8m0_f32_bits(uint32_t x) {
  return x == 0u ? 0x00400000u : (x == 255u ? 0x7fc00000u : x << 23);
}

// 8 E2M1 codes (one 32-bit word: elements 0..7, element 2j in the low nibble
// of byte j) times the fp32 scale sc, as 8 bf16 in element order (gfx950
// converts the two codes of a byte per instruction, low nibble first).
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t w, float sc) {
  const hw_bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const hw_bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const hw_bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const hw_bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// 8 FP8 E4M3 codes (two 32-bit words: elements 0..3 in w0, byte i of a word
// element i) times the fp32 scale sc, as 8 bf16 in element order (gfx950
// converts two codes of a word half per instruction, the low byte first).
// An E4M3 value times a power of two has at most four significant bits, so
// the result is exact while it lies in bf16's normal range.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1, float sc) {
  const hw_bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const hw_bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const hw_bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const hw_bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

}  // namespace cskv
