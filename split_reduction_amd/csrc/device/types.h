// Vector types and raw buffer-resource access for gfx950.
//
// A raw buffer resource carries a base address and a byte bound. A load at an
// offset at or past the bound returns zeros and touches no memory; a store
// there is dropped. That gives predicated loads and stores without branches:
// pass kOOB as the offset when the predicate is false (page
// vllm.models.muse_spark.amd.mono.kernels.dev, ld_vec_if and st_if: an
// out-of-range offset instead of a branch, so the waitcnt pass does not drain
// at a join).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9 raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
// An offset past every bound this library builds (bounds stay below 2^31).
constexpr uint32_t kOOB = 0x80000000u;
// Cache-policy bits of a buffer access on gfx950: bit 1 is NT (streaming).
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;
// SC1: device-scope coherent access. Such a store is written through to the
// level all XCDs share and such a load does not hit a non-coherent copy, so
// they need no cache-wide writeback or invalidate around them (the bits the
// compiler itself emits for relaxed device-scope atomic loads and stores).
constexpr int kPolicyDeviceCoherent = 16;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// 16 bytes at byte offset `off`, or zeros with no memory access when !ok.
template <int POLICY = kPolicyDefault>
__device__ __forceinline__ u32x4 ld16_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : kOOB, 0, POLICY);
}

template <int POLICY = kPolicyDefault>
__device__ __forceinline__ uint32_t ld1_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, ok ? off : kOOB, 0, POLICY);
}

// Stores dropped (no branch) when !ok.
__device__ __forceinline__ void st16_if(bool ok, u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, ok ? off : kOOB, 0, kPolicyDefault);
}
__device__ __forceinline__ void st8_if(bool ok, u32x2 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, ok ? off : kOOB, 0, kPolicyDefault);
}
__device__ __forceinline__ void st4_if(bool ok, uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, ok ? off : kOOB, 0, kPolicyDefault);
}

// Device-scope coherent 16-byte store / load (predicated like the above).
__device__ __forceinline__ void st16_coherent_if(bool ok, u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, ok ? off : kOOB, 0, kPolicyDeviceCoherent);
}
__device__ __forceinline__ u32x4 ld16_coherent_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? off : kOOB, 0, kPolicyDeviceCoherent);
}

// Waits until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace skg
