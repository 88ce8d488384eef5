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

// Piece transpose of a block-scaled weight step across the four lane rows
// (g = lane / 16) of one A row. Natural pieces: lane row g holds the 16
// bytes of elements [g*LK, g*LK + LK) of the step's 4*LK-element window, and
// operand s2 of it is elements g*LK + 8*s2 .. +7. After the transpose,
// operand s2 of lane row g is elements 32*s2 + 8*g .. +7, so that the
// activation operand s2 of all four lane rows is one contiguous 64-byte run
// per token (see the cluster kernel). Each swap exchanges one bit of the
// lane row with one bit of the register index:
//   v_permlane16_swap(a, b): odd rows of a <-> even rows of b (row bit 0),
//   v_permlane32_swap(a, b): rows 2, 3 of a <-> rows 0, 1 of b (row bit 1).
// MXFP4 (eight elements per dword): a 4 x 4 transpose of (lane row, dword).
// MXFP8 (four per dword, operands are dword pairs): a rotation of the three
// bits (lane row, pair) taking group 2*g + p to position (row g, pair p).
template <int WF>
__device__ __forceinline__ u32x4 transpose_pieces(u32x4 v) {
  auto swap16 = [](uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  };
  auto swap32 = [](uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  };
  uint32_t d0 = v[0], d1 = v[1], d2 = v[2], d3 = v[3];
  if constexpr (WF == kMxfp4) {
    swap32(d0, d2);  // row bit 1 <-> dword bit 1
    swap32(d1, d3);
    swap16(d0, d1);  // row bit 0 <-> dword bit 0
    swap16(d2, d3);
  } else {
    swap16(d0, d2);  // row bit 0 <-> pair bit
    swap16(d1, d3);
    swap32(d0, d2);  // row bit 1 <-> pair bit
    swap32(d1, d3);
  }
  return u32x4{d0, d1, d2, d3};
}

}  // namespace skg
