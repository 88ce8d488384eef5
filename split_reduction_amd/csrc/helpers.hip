// Kernels that expose the device helpers on their own, for bit-exact checks:
// bf16 and E4M3 packing, the fixed-order wave sum and the MXFP4 decode. They
// run the same inline helpers the GEMM kernels use.

#include "device/mxfp4.h"
#include "device/wfmt.h"
#include "device/pack.h"
#include "device/types.h"
#include "device/wave.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void pack_bf16_kernel(const float* in, uint32_t* out,
                                                             size_t n) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float2 v = reinterpret_cast<const float2*>(in)[i];
  out[i] = bf16_pair(v.x, v.y);
}

__global__ __launch_bounds__(kThreads) void pack_e4m3_kernel(const float* in, uint32_t* out,
                                                             size_t n) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float4 v = reinterpret_cast<const float4*>(in)[i];
  out[i] = e4m3_pack4(v.x, v.y, v.z, v.w);
}

// One wavefront per group of 64 values; every lane runs the butterfly (the
// grid covers whole wavefronts, so no lane of a wave is inactive).
__global__ __launch_bounds__(kThreads) void wave_sum_kernel(const float* in, float* out,
                                                            size_t n_waves) {
  const size_t wave = (size_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (wave >= n_waves) return;  // uniform across the wave
  const float v = in[wave * 64 + lane];
  out[wave * 64 + lane] = butterfly_sum(v);
}

// One thread per dword of 8 codes: W_out[n, 8i .. 8i+7] = decode(Wq dword i
// of row n, scale of its 32-element block).
__global__ __launch_bounds__(kThreads) void mxfp4_dequant_kernel(const uint32_t* wq,
                                                                 const uint8_t* ws, u32x4* out,
                                                                 int N, int K) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t dwords_per_row = (size_t)K / 8;
  if (i >= (size_t)N * dwords_per_row) return;
  const size_t row = i / dwords_per_row;
  const size_t col = i % dwords_per_row;  // elements 8 col .. 8 col + 7
  const uint32_t code = ws[row * (K / 32) + col / 4];
  const bf16x8 v = fp4x8_bf16(wq[i], e8m0_f32(code));
  out[i] = __builtin_bit_cast(u32x4, v);
}

// One thread per pair of dwords (8 E4M3 codes): W_out[n, 8i .. 8i+7] =
// decode(codes, scale of their 32-element block).
__global__ __launch_bounds__(kThreads) void mxfp8_dequant_kernel(const u32x2* wq,
                                                                 const uint8_t* ws, u32x4* out,
                                                                 int N, int K) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t groups_per_row = (size_t)K / 8;
  if (i >= (size_t)N * groups_per_row) return;
  const size_t row = i / groups_per_row;
  const size_t col = i % groups_per_row;  // elements 8 col .. 8 col + 7
  const uint32_t code = ws[row * (K / 32) + col / 4];
  const u32x2 w = wq[i];
  const bf16x8 v = fp8x8_bf16(w.x, w.y, e8m0_f32(code));
  out[i] = __builtin_bit_cast(u32x4, v);
}

unsigned blocks_for(size_t n, size_t per_block) {
  return (unsigned)((n + per_block - 1) / per_block);
}

}  // namespace

// Zeros n 16-byte pieces with vector stores: the set-up clear of a counter
// area, as a kernel so that a graph that captures it holds no memset node.
__global__ __launch_bounds__(kThreads) void zero16_kernel(u32x4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero16(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned blocks = blocks_for(n, kThreads) < 1024u ? blocks_for(n, kThreads) : 1024u;
  hipLaunchKernelGGL(zero16_kernel, dim3(blocks), dim3(kThreads), 0, s, static_cast<u32x4*>(p), n);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const float* in, uint32_t* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks_for(n, kThreads)), dim3(kThreads), 0, s, in,
                     out, n);
  return hipGetLastError();
}

hipError_t launch_pack_e4m3(const float* in, uint32_t* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_e4m3_kernel, dim3(blocks_for(n, kThreads)), dim3(kThreads), 0, s, in,
                     out, n);
  return hipGetLastError();
}

// Reference stream: every byte of src read once with coalesced 16-byte
// non-temporal loads. Workgroup b reads one contiguous block (its CU then
// walks DRAM pages in order), its 512 lanes on consecutive 16-byte pieces,
// four loads in flight per lane, 1024 workgroups: the fastest of the
// configurations measured (1024 x 512 x 4 with the hint: 29 MB in 6.2 us,
// 537 MB at 6.9 TB/s; 512 x 1024 x 8 without it: 6.6 us, 5.8 TB/s). The
// words are folded into one per workgroup that is stored only if it equals
// a value no input of the probe produces, so the loads stay live without
// output traffic.
constexpr int kReadProbeThreads = 512;
constexpr int kReadProbeLoads = 4;
__global__ __launch_bounds__(kReadProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                       uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;  // pieces per workgroup
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  constexpr int TH = kReadProbeThreads;
  uint32_t acc = 0;
  for (size_t i = lo + threadIdx.x; i < hi; i += kReadProbeLoads * TH) {
    u32x4 v[kReadProbeLoads];
#pragma unroll
    for (int u = 0; u < kReadProbeLoads; ++u)
      v[u] = (i + u * TH < hi) ? __builtin_nontemporal_load(src + i + u * TH) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kReadProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kReadProbeMagic) sink[blockIdx.x % kReadProbeSinkWords] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  if (bytes < 16) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(kReadProbeThreads), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_wave_sum(const float* in, float* out, size_t n_waves, hipStream_t s) {
  if (n_waves == 0) return hipSuccess;
  hipLaunchKernelGGL(wave_sum_kernel, dim3(blocks_for(n_waves, kThreads / 64)), dim3(kThreads), 0,
                     s, in, out, n_waves);
  return hipGetLastError();
}

hipError_t launch_mxfp4_dequant(const void* wq, const void* ws, void* out, int N, int K,
                                hipStream_t s) {
  const size_t n = (size_t)N * (size_t)(K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3(blocks_for(n, kThreads)), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(wq), static_cast<const uint8_t*>(ws),
                     static_cast<u32x4*>(out), N, K);
  return hipGetLastError();
}

hipError_t launch_mxfp8_dequant(const void* wq, const void* ws, void* out, int N, int K,
                                hipStream_t s) {
  const size_t n = (size_t)N * (size_t)(K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_dequant_kernel, dim3(blocks_for(n, kThreads)), dim3(kThreads), 0, s,
                     static_cast<const u32x2*>(wq), static_cast<const uint8_t*>(ws),
                     static_cast<u32x4*>(out), N, K);
  return hipGetLastError();
}

}  // namespace skg
