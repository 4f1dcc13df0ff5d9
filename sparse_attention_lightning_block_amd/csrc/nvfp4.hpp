// NVFP4 key decoding on gfx950.
//
// Format ([listing] "nvfp4-megamoe-kernel -- .../indexer_score_topk.cu", NVFP4 notes
// and dequant_fp4_scalar; [commits] 79ef87f9a9 and e74c84458c): element d of a key
// is the low nibble of byte d/2 for even d and the high nibble for odd d; bit 3 of
// the nibble is the sign and bits 2..0 select the magnitude 0, .5, 1, 1.5, 2, 3, 4
// or 6 (E2M1, exponent bias 1); every 16 consecutive elements share one OCP FP8
// E4M3 scale byte.  The code value E2M1 * E4M3 has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16 and in fp32.
//
// gfx950 converts E2M1 pairs with v_cvt_scalef32_pk_{f16,f32}_fp4.  That
// instruction applies only the exponent of its fp32 scale operand, so it is used
// with scale 1.0 and the E4M3 scale (decoded exactly by v_cvt_f32_fp8) is applied
// with a separate multiply, which is exact because the product is representable.
#pragma once

#include "common.hpp"

namespace salb {

// OCP E4M3 byte -> fp32 (exact; 0x7f/0xff give NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Four bytes (eight E2M1 codes, element order low nibble first) times one E4M3
// scale -> eight fp16 code values packed as an MFMA operand (element i of the
// result is element i of the word).
__device__ __forceinline__ half8v decode8_f16(uint32_t word, half2v s2) {
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * s2;
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * s2;
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * s2;
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * s2;
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, a);
  r[1] = __builtin_bit_cast(uint32_t, b);
  r[2] = __builtin_bit_cast(uint32_t, c);
  r[3] = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(half8v, r);
}

__device__ __forceinline__ half2v splat_scale_f16(uint32_t byte) {
  _Float16 s = (_Float16)e4m3_to_f32(byte);  // exact: every E4M3 value is an fp16 value
  half2v r = {s, s};
  return r;
}

// Four bytes (eight E2M1 codes) times one E4M3 scale -> eight exact fp32 code values.
__device__ __forceinline__ void decode8_f32(uint32_t word, float scale, float* out) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float2v v;
    switch (b) {
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
    }
    out[2 * b] = v[0] * scale;
    out[2 * b + 1] = v[1] * scale;
  }
}

}  // namespace salb
