// The output stage of a GEMM launch: C as bf16 (round to nearest even, page
// vllm.models.muse_spark.amd.mono.kernels.dev, bf16_pair) or as OCP E4M3FN
// bytes (page vllm.models.deepseek_v41.amd.mono.common.ops, fp8_pack4): the
// FP32 sum times the caller's scale, saturated to +-448 so that every value is
// in the packing helper's range, then rounded to nearest even.
//
// Kernels address C by element index (token * N + feature); the element size
// comes from here.
#pragma once

#include "pack.h"
#include "types.h"
#include "../skgemm_internal.h"

namespace skg {

struct COut {
  rsrc_t r;
  bool e4m3;
  float scale;
};

__device__ __forceinline__ COut make_cout(const GemmParams& p) {
  COut o;
  o.e4m3 = p.out_e4m3 != 0;
  o.scale = p.c_scale;
  o.r = make_rsrc(p.c, (uint32_t)p.T * (uint32_t)p.N * (o.e4m3 ? 1u : 2u));
  return o;
}

// x * scale clamped to the E4M3FN range (finite inputs).
__device__ __forceinline__ float e4m3_in_range(float x, float scale) {
  return fminf(fmaxf(x * scale, -448.0f), 448.0f);
}

// Four consecutive outputs of one token, element index `el` (el % 4 == 0).
// POL: the stores' cache policy (device-coherent where another CU reads C
// within the same launch).
template <int POL = kPolicyDefault>
__device__ __forceinline__ void store_quad(const COut& o, bool ok, f32x4 v, uint32_t el) {
  if (o.e4m3) {
    const uint32_t w = e4m3_pack4(e4m3_in_range(v.x, o.scale), e4m3_in_range(v.y, o.scale),
                                  e4m3_in_range(v.z, o.scale), e4m3_in_range(v.w, o.scale));
    __builtin_amdgcn_raw_buffer_store_b32(w, o.r, ok ? el : kOOB, 0, POL);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(bf16_quad(v), o.r, ok ? el * 2u : kOOB, 0, POL);
  }
}

// Two consecutive outputs of one token, element index `el` (el % 2 == 0).
template <int POL = kPolicyDefault>
__device__ __forceinline__ void store_pair(const COut& o, bool ok, float a, float b, uint32_t el) {
  if (o.e4m3) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_in_range(a, o.scale), e4m3_in_range(b, o.scale), 0, false);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w & 0xFFFF), o.r, ok ? el : kOOB, 0, POL);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(bf16_pair(a, b), o.r, ok ? el * 2u : kOOB, 0, POL);
  }
}

}  // namespace skg
