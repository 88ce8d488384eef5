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
// An offset at or past every bound this library builds. The host keeps each
// resource's span at most 2^31 bytes: per-tile resources by the size limits
// (at most 256 rows of at most 2^23 bytes), whole-matrix resources by an
// explicit check where the kernel that uses them is chosen.
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

template <int POLICY = kPolicyDefault>
__device__ __forceinline__ u32x2 ld8_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, ok ? off : kOOB, 0, POLICY);
}
template <int POLICY = kPolicyDefault>
__device__ __forceinline__ uint32_t ld4_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, ok ? off : kOOB, 0, POLICY);
}
template <int POLICY = kPolicyDefault>
__device__ __forceinline__ uint32_t ld2_if(bool ok, rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, ok ? off : kOOB, 0, POLICY);
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

// Whole-line weight loads. A v_mfma_f32_16x16x32 A operand holds, in lane
// (li = lane % 16, g = lane / 16), 16 bytes of row li at K block g, so a load
// straight into operand layout covers 16 rows x 64 bytes: half of each
// 128-byte line, and streaming such halves reaches ~4.9 TB/s where whole
// lines with the non-temporal hint reach ~6.4 TB/s (measured, 264 MB). The
// pair below loads rows 0-7 (load 0) and rows 8-15 (load 1) instead, lane
// (li, g) taking row li % 8 + 8 * load at 64-byte window li / 8, block g:
// 8 whole lines per instruction. One DPP move per register (rotate by 8
// lanes inside each 16-lane row, written to half the lanes) turns the pair
// into the two 16-row operands, of windows 0 and 1.
//
// Byte offset of lane (li, g) within load 0, relative to row 0, window 0.
__device__ __forceinline__ uint32_t line_pair_offset(int li, int g, uint32_t row_bytes) {
  return (uint32_t)(li & 7) * row_bytes + 64u * (uint32_t)(li >> 3) + 16u * (uint32_t)g;
}
__device__ __forceinline__ void line_pair_to_operands(u32x4 l0, u32x4 l1, u32x4& w0, u32x4& w1) {
  constexpr int kRowRor8 = 0x128;  // DPP row_ror:8
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // Lanes 8-15 of each row (banks 2, 3) take load 1's rows 8-15, window 0.
    w0[e] = (uint32_t)__builtin_amdgcn_update_dpp((int)l0[e], (int)l1[e], kRowRor8, 0xF, 0xC, false);
    // Lanes 0-7 (banks 0, 1) take load 0's rows 0-7, window 1.
    w1[e] = (uint32_t)__builtin_amdgcn_update_dpp((int)l1[e], (int)l0[e], kRowRor8, 0xF, 0x3, false);
  }
}

// Compiler-only ordering point of the split-K hand-offs. Their counters are
// relaxed device-scope atomics and their partials device-coherent buffer
// accesses; the hardware order between the two comes from s_waitcnt (stores
// complete before the arrival is issued) and from data dependence (partials
// are loaded only after a branch on the counter's value). A relaxed atomic
// does not stop the compiler from moving other memory accesses across it, so
// each side of the hand-off puts this fence between the two.
__device__ __forceinline__ void handoff_order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Waits until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima). The wait
// intrinsic itself is not a memory operation to the compiler, so fences on
// both sides keep every access on its side of the wait.
__device__ __forceinline__ void wait_vmem_all() {
  handoff_order();
  __builtin_amdgcn_s_waitcnt(0x0F70);
  handoff_order();
}

}  // namespace skg
