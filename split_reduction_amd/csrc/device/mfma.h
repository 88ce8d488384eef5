// v_mfma_f32_16x16x32_bf16 (page vllm.models.muse_spark.amd.mono.kernels.dev,
// mfma_bf16: a, b bf16x8, c f32x4).
//
// Operand layout on gfx950, lane l = 16*g + i (g = l / 16, i = l % 16):
//   A (16 x 32): lane l holds 8 K-consecutive elements of row i, the K block g.
//   B (32 x 16): lane l holds 8 K-consecutive elements of column i, block g.
//   D (16 x 16): lane l holds rows 4*g .. 4*g+3 of column i.
// Only the pairing matters for the contraction: any permutation of K applied
// to both A and B leaves the product unchanged, which lets one 16-byte load
// of a weight row be one A operand. With A = weights (rows = output features
// n) and B = activations (columns = tokens t), D lane l holds
// C[t = i][n = 4*g .. 4*g+3]: row r, token t sits in lane 16*(r/4) + t,
// element r % 4 (page vllm.models.deepseek_v41.amd.mono.common.ops, row_sum).
#pragma once

#include "types.h"

namespace skg {

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace skg
