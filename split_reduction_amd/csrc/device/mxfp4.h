// MXFP4 decode: E2M1 elements with one E8M0 power-of-two scale per 32.
//
// e8m0_f32: the biased exponent c (1..254) shifted into the float32 exponent
// field is exactly 2^(c-127) (page vllm.models.muse_spark.amd.mono.kernels.dev,
// e8m0_f32).
//
// fp4x8_bf16: one dword holds eight E2M1 codes, element j in bits 4j..4j+3
// (low nibble first). v_cvt_scalef32_pk_bf16_fp4 turns the two codes of the
// selected byte into two bf16 values times the float32 scale, the low nibble
// into the low half; four byte selects give the eight values in order (same
// page, fp4x8_bf16). Every E2M1 value has at most two significant bits, so
// the product with a power of two is exact in bf16 whenever it stays normal.
#pragma once

#include "types.h"

namespace skg {

__device__ __forceinline__ float e8m0_f32(uint32_t code) { return __uint_as_float(code << 23); }

__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t word, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

}  // namespace skg
