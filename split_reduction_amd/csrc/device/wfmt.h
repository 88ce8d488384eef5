// Weight formats of the GEMM kernels and their in-register decode.
//
//   kBf16   bf16 weights, used as they are.
//   kMxfp4  E2M1 codes (two per byte, low nibble first) with one E8M0 scale
//           per 32 K elements (page vllm.models.muse_spark.amd.mono.kernels.dev,
//           fp4x8_bf16 and e8m0_f32).
//   kMxfp8  OCP E4M3FN codes (one per byte) with one E8M0 scale per 32 K
//           elements: the same block scaling with eight-bit elements. Every
//           E4M3 value has at most four significant bits, so its product with
//           a power of two is exact in bf16 wherever it stays normal.
//
// A lane loads 16 bytes of one weight row per load step: 32 E2M1 or 16 E4M3
// codes, consecutive in K and inside one scale block, decoded into 4 or 2
// MFMA operands of 8 elements; bf16 lanes load C pieces of 8 elements.
#pragma once

#include "mxfp4.h"
#include "types.h"

namespace skg {

constexpr int kBf16 = 0;
constexpr int kMxfp4 = 1;
constexpr int kMxfp8 = 2;

// K elements of one lane's 16-byte piece.
constexpr int lane_k(int wf) { return wf == kMxfp4 ? 32 : wf == kMxfp8 ? 16 : 8; }

// Bytes of a weight row of K elements, and the byte offset of element k in it.
constexpr uint32_t row_bytes(int wf, uint32_t K) {
  return wf == kMxfp4 ? K / 2 : wf == kMxfp8 ? K : 2 * K;
}
constexpr uint32_t elem_byte(int wf, uint32_t k) {
  return wf == kMxfp4 ? k / 2 : wf == kMxfp8 ? k : 2 * k;
}

// Weight bytes per K element, for host-side traffic estimates.
constexpr double weight_bytes_per_elem(int wf) {
  return wf == kMxfp4 ? 0.5 + 1.0 / 32 : wf == kMxfp8 ? 1.0 + 1.0 / 32 : 2.0;
}

// Eight E4M3 codes (lo: elements 0..3 low byte first, hi: 4..7) times the
// float32 scale as one bf16x8 operand. v_cvt_scalef32_pk_bf16_fp8 converts
// the two codes of the selected 16-bit half, the lower byte into the lower
// half of the result.
__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t lo, uint32_t hi, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// MFMA operand s2 of a scaled format's 16-byte piece v (elements 8*s2 .. +7).
template <int WF>
__device__ __forceinline__ bf16x8 decode_operand(u32x4 v, int s2, float scale) {
  if constexpr (WF == kMxfp4) {
    return fp4x8_bf16(v[s2], scale);
  } else {
    return fp8x8_bf16(v[2 * s2], v[2 * s2 + 1], scale);
  }
}

}  // namespace skg
