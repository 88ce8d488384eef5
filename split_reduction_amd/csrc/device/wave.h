// Wavefront (64-lane) exchanges and the fixed-order butterfly sum.
//
// xshfl<OFF>(v): the value of lane (lane ^ OFF). In-row offsets use DPP moves
// (VALU latency, no LDS): 1 and 2 are quad permutations; 4 and 8 combine a
// row shift right into the upper banks with a row shift left into the lower
// banks of each 16-lane row. Offsets 16 and 32 cross rows and use
// v_permlane16_swap / v_permlane32_swap (page
// vllm.models.deepseek_v41.amd.mono.common.ops, xshfl and permlane_swap).
//
// xred<OFF>(v) = v + v[lane ^ OFF] in FP32. For 16 and 32 one swap of v with
// itself yields both halves at once (same page, xred): after
// permlane32_swap(v, v) the first result holds v's lower half in both halves
// and the second v's upper half, so their sum is v + v[lane ^ 32] everywhere.
//
// butterfly_sum(v): xred over 32, 16, 8, 4, 2, 1 in that order; the order is
// the numerical contract (same page, butterfly), so every lane ends with the
// same bits and repeated runs agree.
#pragma once

#include "types.h"

namespace skg {

// DPP controls (ISA encodings): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_shl:n = 0x100 + n, row_shr:n = 0x110 + n. Bank masks pick 4-lane banks.
template <int OFF>
__device__ __forceinline__ int xshfl_dpp(int x) {
  static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8, "in-row offsets only");
  if constexpr (OFF == 1) {
    return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (OFF == 2) {
    return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (OFF == 4) {
    int y = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xA, false);  // banks 1,3 <- lane-4
    return __builtin_amdgcn_update_dpp(y, x, 0x104, 0xF, 0x5, false);   // banks 0,2 <- lane+4
  } else {
    int y = __builtin_amdgcn_update_dpp(x, x, 0x118, 0xF, 0xC, false);  // banks 2,3 <- lane-8
    return __builtin_amdgcn_update_dpp(y, x, 0x108, 0xF, 0x3, false);   // banks 0,1 <- lane+8
  }
}

template <int OFF>
__device__ __forceinline__ float xred_add(float v) {
  if constexpr (OFF >= 16) {
    int x = __float_as_int(v);
    auto p = (OFF == 32) ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                         : __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return __int_as_float(p[0]) + __int_as_float(p[1]);
  } else {
    return v + __int_as_float(xshfl_dpp<OFF>(__float_as_int(v)));
  }
}

__device__ __forceinline__ float butterfly_sum(float v) {
  v = xred_add<32>(v);
  v = xred_add<16>(v);
  v = xred_add<8>(v);
  v = xred_add<4>(v);
  v = xred_add<2>(v);
  v = xred_add<1>(v);
  return v;
}

}  // namespace skg
