// Bit-exact packing helpers.
//
// bf16: round to nearest even on the float32 bit pattern, two values to one
// word with the first in the low half (page
// vllm.models.muse_spark.amd.mono.kernels.dev, bf16_pair). Written as integer
// arithmetic so the result does not depend on the float mode registers:
// adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
// when the dropped half exceeds one half unit, or equals it with an odd kept
// half. NaN keeps its sign and top payload bits and is made quiet.
//
// E4M3: v_cvt_pk_fp8_f32 on gfx950 converts to OCP E4M3FN with round to
// nearest even; two calls fill the low then the high 16 bits (page
// vllm.models.deepseek_v41.amd.mono.common.ops, fp8_pack4: bytes a, b, c, d
// from the low byte; inputs already in range, |x| <= 448).
#pragma once

#include "types.h"

namespace skg {

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Four float32 -> four bf16 in two words (element 0 in the low half of word 0).
__device__ __forceinline__ u32x2 bf16_quad(f32x4 v) {
  u32x2 w;
  w.x = bf16_pair(v.x, v.y);
  w.y = bf16_pair(v.z, v.w);
  return w;
}

// Packed bf16 word -> the float32 of its low / high half (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

}  // namespace skg
