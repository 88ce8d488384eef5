// C ABI of libskgemm.so: argument checks, split-K workspace ownership, token
// blocking and kernel dispatch. Declarations and contracts: include/skgemm.h.

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "skgemm.h"
#include "skgemm_internal.h"
#include "device/wfmt.h"

namespace {

constexpr int kTokenBlock = 128;  // rows of X / C per launch (16 * 8 MFMA tiles)

thread_local int g_last_hip_error = 0;

// Pinned choices (skgemm_set_override), stored as value + 1: 0 (the initial
// state) means the library's own choice.
std::atomic<int> g_knobs[skg::kKnobCount];

// The split-K hand-off of the persistent kernel unless a test pins one:
// 0 arrival counter, 1 tagged mailbox.
constexpr int kDefaultHandoff = 0;
using skg::knob;

// How long a tile's owner waits for the other split ranks before handing the
// tile to the last to arrive: 100 us of the 100 MHz device clock unless a
// test pins another tick count (0 exercises the hand-over path).
uint32_t owner_wait_ticks() { return (uint32_t)skg::knob(skg::kKnobOwnerWait, 10000); }

// Optional phase-stamp buffer (skgemm_set_timeline).
std::atomic<uint64_t*> g_stamps{nullptr};
std::atomic<size_t> g_stamps_cap{0};

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return SKGEMM_EHIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// K granularity of one split rank's slice per weight format: a load step of
// 32 bf16 elements, or four lanes' 16-byte pieces of block-scaled codes.
int k_step(int wf) { return wf == skg::kBf16 ? 32 : 4 * skg::lane_k(wf); }

// Argument checks shared by the GEMM entry points and the tactic query.
// Pointers are checked only when check_ptrs is set.
int check_gemm(int wf, const void* w, const void* ws, const void* x, const void* c, int T, int N,
               int K, int S, bool check_ptrs) {
  const bool mx = wf != skg::kBf16;
  if (T < 0 || N < 0 || K < 0) return SKGEMM_EINVAL;
  if (S != 1 && S != 2 && S != 4 && S != 8) return SKGEMM_EINVAL;
  if (N % 16 != 0) return SKGEMM_ESHAPE;
  if (K % (k_step(wf) * S) != 0) return SKGEMM_ESHAPE;
  if (N > SKGEMM_MAX_N || K > SKGEMM_MAX_K) return SKGEMM_ESHAPE;
  if (!check_ptrs || T == 0 || N == 0) return SKGEMM_OK;
  if (c == nullptr) return SKGEMM_EINVAL;
  if (!aligned16(c)) return SKGEMM_EALIGN;
  if (K > 0) {
    if (w == nullptr || x == nullptr || (mx && ws == nullptr)) return SKGEMM_EINVAL;
    if (!aligned16(w) || !aligned16(x)) return SKGEMM_EALIGN;
  }
  return SKGEMM_OK;
}

// ---- split-K workspace: one per (device, stream) ---------------------------

struct Workspace {
  float* part = nullptr;
  size_t part_bytes = 0;
  uint32_t* cnt = nullptr;  // cnt_count counters, then kHealthWords health words
  size_t cnt_count = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Workspaces replaced by larger ones, kept until skgemm_release: a HIP graph
// captured earlier still names their addresses in its kernel arguments, so
// freeing them would let a later replay write into memory handed out again.
std::vector<std::pair<int, Workspace>> g_retired;

// Makes the stream's workspace hold at least part_bytes of partials and
// cnt_count zeroed counters. Growing allocates new buffers and retires the old
// ones (kept allocated until skgemm_release); under graph capture it refuses
// instead.
int ensure_workspace(hipStream_t stream, size_t part_bytes, size_t cnt_count, Workspace* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  // A new entry holds nothing yet (a call asking for no bytes still needs the
  // counter, health and synchronisation words).
  if (w.cnt != nullptr && w.part_bytes >= part_bytes && w.cnt_count >= cnt_count) {
    *out = w;
    return SKGEMM_OK;
  }
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e);
  if (st != hipStreamCaptureStatusNone) return SKGEMM_ENOMEM;
  Workspace nw;
  nw.part_bytes = std::max(part_bytes, (size_t)256);
  nw.cnt_count = std::max(cnt_count, (size_t)64);
  if (hipMalloc((void**)&nw.part, nw.part_bytes) != hipSuccess) return SKGEMM_ENOMEM;
  const size_t words = nw.cnt_count + skg::kHealthWords + skg::kSyncWords;
  if (hipMalloc((void**)&nw.cnt, words * sizeof(uint32_t)) != hipSuccess) {
    (void)hipFree(nw.part);
    return SKGEMM_ENOMEM;
  }
  e = hipMemsetAsync(nw.cnt, 0, words * sizeof(uint32_t), stream);
  // Partials start zeroed: a mailbox tag is never 0, so no slot of a new
  // workspace can hold a value that passes for this launch's.
  if (e == hipSuccess) e = hipMemsetAsync(nw.part, 0, nw.part_bytes, stream);
  if (e != hipSuccess) {
    (void)hipFree(nw.part);
    (void)hipFree(nw.cnt);
    return hip_fail(e);
  }
  if (w.part != nullptr || w.cnt != nullptr) g_retired.emplace_back(dev, w);
  w = nw;
  *out = w;
  return SKGEMM_OK;
}

size_t part_bytes_for(int T, int N, int S) {
  return (size_t)S * (size_t)std::min(T, kTokenBlock) * (size_t)N * sizeof(float);
}
// Arrival counters, one per 16 output rows, kCntStride words apart.
size_t counters_for(int N) { return (size_t)N / 16 * skg::kCntStride; }

// Compute units of the current device (the owner wait is used only while the
// whole grid fits on them).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  cache[dev] = n;
  return n;
}

// A batch of L problems of one shape; strides in bytes (problem l of W at
// w + l * bw, and so on).
struct Batch {
  int L = 1;
  uint64_t bw = 0, bws = 0, bx = 0, bc = 0;
};

int check_batch(const Batch& b, int T, int N) {
  if (b.L < 1 || b.L > SKGEMM_MAX_BATCH) return SKGEMM_EINVAL;
  if (b.L == 1) return SKGEMM_OK;
  if ((b.bw | b.bx | b.bc) % 16 != 0) return SKGEMM_EALIGN;  // Wscale needs no alignment
  if (b.bc < (uint64_t)T * (uint64_t)N * 2) return SKGEMM_EINVAL;  // outputs must not overlap
  return SKGEMM_OK;
}

// `given`: a workspace the caller provides (the no-allocation entry point's
// fixed scratch); calls that need more than it holds get SKGEMM_ESCRATCH.
// Without it the stream's own workspace is used (allocated or grown here).
// Output format of a call: bf16, or E4M3FN bytes of sum * c_scale (saturated).
struct OutFmt {
  int e4m3 = 0;
  float c_scale = 1.0f;
};

int run_gemm(int wf, const void* w, const void* ws, const void* x, void* c, int T, int N, int K,
             int S, hipStream_t stream, const Batch& batch = Batch{}, const Workspace* given = nullptr,
             const OutFmt& out = OutFmt{}) {
  int rc = check_gemm(wf, w, ws, x, c, T, N, K, S, true);
  if (rc != SKGEMM_OK) return rc;
  rc = check_batch(batch, T, N);
  if (rc != SKGEMM_OK) return rc;
  if (T == 0 || N == 0) return SKGEMM_OK;
  const int L = batch.L;
  // The tagged-mailbox hand-off (persistent kernel, single problems with a
  // split, not in the no-allocation scratch) stores 8 bytes per partial.
  bool mailbox = false;
  if (S > 1 && L == 1 && given == nullptr && knob(skg::kKnobHandoff, kDefaultHandoff) == 1) {
    skg::Tactic t0{};
    mailbox = skg::pick_tactic(std::min(kTokenBlock, T), N, K, S, wf, &t0, L) && skg::tactic_mailbox(t0);
  }
  Workspace wsp;
  if (S > 1) {
    const size_t part = part_bytes_for(T, N, S) * (size_t)L * (mailbox ? 2 : 1), cnts = counters_for(N) * (size_t)L;
    if (given != nullptr) {
      if (part > given->part_bytes || cnts > given->cnt_count) return SKGEMM_ESCRATCH;
      wsp = *given;
    } else {
      rc = ensure_workspace(stream, part, cnts, &wsp);
      if (rc != SKGEMM_OK) return rc;
    }
  }
  const int cus = device_cus();
  for (int t0 = 0; t0 < T; t0 += kTokenBlock) {
    const int tb = std::min(kTokenBlock, T - t0);
    skg::Tactic tac{};
    if (!skg::pick_tactic(tb, N, K, S, wf, &tac, L)) return SKGEMM_ESHAPE;
    skg::GemmParams p{};
    p.w = w;
    p.wscale = static_cast<const uint8_t*>(ws);
    p.x = static_cast<const uint8_t*>(x) + (size_t)t0 * (size_t)K * 2;
    p.c = static_cast<uint8_t*>(c) + (size_t)t0 * (size_t)N * (out.e4m3 ? 1 : 2);
    p.out_e4m3 = out.e4m3;
    p.c_scale = out.c_scale;
    p.part = wsp.part;
    p.cnt = wsp.cnt;
    p.T = tb;
    p.N = N;
    p.K = K;
    p.S = S;
    p.ks = K / S;
    p.kc = tac.kc;
    p.nchunks = (tac.kc > 0) ? p.ks / tac.kc : 0;
    p.stamps = ((size_t)tac.grid * 8 <= g_stamps_cap.load()) ? g_stamps.load() : nullptr;
    // Owners wait for their peers only while every workgroup of the launch can
    // be resident at once; beyond, they hand their tiles over at once.
    const bool all_resident =
        tac.resident > 0 && cus > 0 && (long)tac.grid * L <= (long)cus * tac.resident;
    p.owner_wait = all_resident ? owner_wait_ticks() : 0u;
    p.pdefer = tac.pdefer;
    p.health = wsp.cnt != nullptr ? wsp.cnt + wsp.cnt_count : nullptr;
    p.mailbox = (mailbox && skg::tactic_mailbox(tac)) ? 1 : 0;
    p.epoch = wsp.cnt != nullptr ? p.health + skg::kHealthWords + skg::kEpochWord : nullptr;
    p.L = L;
    p.bw = batch.bw;
    p.bws = batch.bws;
    p.bx = batch.bx;
    p.bc = batch.bc;
    p.bpart = (uint64_t)S * (uint64_t)tb * (uint64_t)N;
    p.bcnt = (uint32_t)counters_for(N);
    hipError_t e = skg::launch_gemm(tac, p, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return SKGEMM_OK;
}

// ---- the fixed scratch of skgemm_bf16_noalloc -----------------------------
// One array per GPU, held until the process ends: arrival counters for the
// largest N (one 128-byte line per 16 output rows) and the health words at
// the front, FP32 partials after them. In host code `scratch` names a host
// stand-in, not device memory: every use goes through the device address
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchCounterWords = (size_t)SKGEMM_MAX_N / 16 * skg::kCntStride;
constexpr size_t kScratchPartOffset = SKGEMM_NOALLOC_PART_OFFSET;
static_assert(kScratchCounterWords * 4 + skg::kHealthWords * 4 <= kScratchPartOffset,
              "counters and health words fit before the partials");
static_assert(kScratchPartOffset % 256 == 0 && SKGEMM_NOALLOC_SCRATCH_BYTES > kScratchPartOffset,
              "partials start on a 256-byte boundary inside the scratch");

static __device__ __align__(256) uint8_t scratch[SKGEMM_NOALLOC_SCRATCH_BYTES];

struct ScratchState {
  uint8_t* ptr = nullptr;  // device address of this GPU's copy of `scratch`
  bool zeroed = false;     // its counter area was cleared outside graph capture
};
std::mutex g_scratch_mu;
std::map<int, ScratchState> g_scratch;

// The current device's scratch as a workspace. At the first call on a device
// its address is looked up; until one call has cleared the counter area
// outside graph capture, each call first enqueues that clear (a fill kernel,
// no memset node in a captured graph); the first uncaptured clear is waited
// for, so calls on other streams start from zeroed counters.
int noalloc_workspace(hipStream_t stream, Workspace* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& st = g_scratch[dev];
  if (st.ptr == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    st.ptr = static_cast<uint8_t*>(ptr);
  }
  if (!st.zeroed) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e);
    e = skg::launch_zero16(st.ptr, kScratchPartOffset, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (cap == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e);
      st.zeroed = true;
    }
  }
  out->cnt = reinterpret_cast<uint32_t*>(st.ptr);
  out->cnt_count = kScratchCounterWords;
  out->part = reinterpret_cast<float*>(st.ptr + kScratchPartOffset);
  out->part_bytes = SKGEMM_NOALLOC_SCRATCH_BYTES - kScratchPartOffset;
  return SKGEMM_OK;
}

}  // namespace

int skg::knob(int k, int dflt) {
  if (k < 0 || k >= skg::kKnobCount) return dflt;
  const int v = g_knobs[k].load(std::memory_order_relaxed);
  return v == 0 ? dflt : v - 1;
}

extern "C" {

SKGEMM_API int skgemm_bf16(const void* W, const void* X, void* C, int T, int N, int K,
                           int split_k, hipStream_t stream) {
  return run_gemm(skg::kBf16, W, nullptr, X, C, T, N, K, split_k, stream);
}

SKGEMM_API int skgemm_bf16_e4m3(const void* W, const void* X, void* C8, float c_scale, int T, int N,
                                int K, int split_k, hipStream_t stream) {
  if (!(c_scale > 0.0f) || !(c_scale < 3.0e38f)) return SKGEMM_EINVAL;  // finite, positive (NaN fails)
  OutFmt out;
  out.e4m3 = 1;
  out.c_scale = c_scale;
  return run_gemm(skg::kBf16, W, nullptr, X, C8, T, N, K, split_k, stream, Batch{}, nullptr, out);
}

SKGEMM_API int skgemm_bf16_chain(const void* const* W, const void* X, void* const* C, const int* dims,
                                 int L, int T, int split_k, hipStream_t stream) {
  if (W == nullptr || C == nullptr || dims == nullptr || X == nullptr) return SKGEMM_EINVAL;
  if (L < 1 || L > SKGEMM_MAX_CHAIN || T < 1 || T > 16) return SKGEMM_EINVAL;
  if (split_k != 1 && split_k != 2 && split_k != 4 && split_k != 8) return SKGEMM_EINVAL;
  for (int i = 0; i <= L; ++i) {
    if (dims[i] < 1) return SKGEMM_EINVAL;
    if (dims[i] > SKGEMM_MAX_K || dims[i] > SKGEMM_MAX_N) return SKGEMM_ESHAPE;
  }
  if (!aligned16(X)) return SKGEMM_EALIGN;
  const int cus = device_cus();
  skg::ChainParams p{};
  for (int i = 0; i < L; ++i) {
    if (W[i] == nullptr || C[i] == nullptr) return SKGEMM_EINVAL;
    if (!aligned16(W[i]) || !aligned16(C[i])) return SKGEMM_EALIGN;
    if (dims[i] % (32 * split_k) != 0 || dims[i + 1] % 16 != 0) return SKGEMM_ESHAPE;
    // K folded two ways (8-row tiles) where 16-row tiles would leave CUs
    // idle and the tokens fit in half an MFMA operand.
    p.fold[i] = (T <= 8 && dims[i + 1] / 16 < (cus > 0 ? cus : 256) && dims[i] % (64 * split_k) == 0) ? 2 : 1;
    // C[i] must not overlap the activations it is computed from.
    const uintptr_t a0 = (uintptr_t)(i == 0 ? X : C[i - 1]);
    const uintptr_t a1 = a0 + (uintptr_t)T * (uintptr_t)dims[i] * 2;
    const uintptr_t c0 = (uintptr_t)C[i], c1 = c0 + (uintptr_t)T * (uintptr_t)dims[i + 1] * 2;
    if (c0 < a1 && a0 < c1) return SKGEMM_EINVAL;
  }
  Workspace wsp;
  int rc = ensure_workspace(stream, 0, 0, &wsp);
  if (rc != SKGEMM_OK) return rc;
  if (wsp.cnt == nullptr) return SKGEMM_ENOMEM;  // the barrier words must exist
  for (int i = 0; i < L; ++i) {
    p.w[i] = W[i];
    p.c[i] = C[i];
  }
  for (int i = 0; i <= L; ++i) p.dims[i] = dims[i];
  p.x = X;
  p.L = L;
  p.T = T;
  p.S = split_k;
  p.health = wsp.cnt + wsp.cnt_count;
  p.sync = p.health + skg::kHealthWords;
  p.wait_ticks = 20000000u;  // 200 ms: a barrier wait that long means something is broken
  if (cus <= 0) return hip_fail(hipErrorInvalidDevice);
  const hipError_t e = skg::launch_chain(p, cus, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_bf16_noalloc(const void* W, const void* X, void* C, int T, int N, int K,
                                   int split_k, hipStream_t stream) {
  // Shape checks first: a call the scratch cannot serve fails before any
  // device work (the same checks run_gemm repeats).
  int rc = check_gemm(skg::kBf16, W, nullptr, X, C, T, N, K, split_k, true);
  if (rc != SKGEMM_OK) return rc;
  if (T == 0 || N == 0) return SKGEMM_OK;
  if (split_k > 1 && part_bytes_for(T, N, split_k) > SKGEMM_NOALLOC_SCRATCH_BYTES - kScratchPartOffset)
    return SKGEMM_ESCRATCH;
  Workspace w;
  if (split_k > 1) {
    rc = noalloc_workspace(stream, &w);
    if (rc != SKGEMM_OK) return rc;
  }
  return run_gemm(skg::kBf16, W, nullptr, X, C, T, N, K, split_k, stream, Batch{}, &w);
}

SKGEMM_API int skgemm_mxfp4(const void* Wq, const void* Wscale, const void* X, void* C, int T,
                            int N, int K, int split_k, hipStream_t stream) {
  return run_gemm(skg::kMxfp4, Wq, Wscale, X, C, T, N, K, split_k, stream);
}

SKGEMM_API int skgemm_mxfp8(const void* Wq8, const void* Wscale, const void* X, void* C, int T,
                            int N, int K, int split_k, hipStream_t stream) {
  return run_gemm(skg::kMxfp8, Wq8, Wscale, X, C, T, N, K, split_k, stream);
}

SKGEMM_API int skgemm_bf16_batched(const void* W, const void* X, void* C, int T, int N, int K,
                                   int split_k, int L, size_t w_stride, size_t x_stride,
                                   size_t c_stride, hipStream_t stream) {
  Batch b;
  b.L = L;
  b.bw = w_stride;
  b.bx = x_stride;
  b.bc = c_stride;
  return run_gemm(skg::kBf16, W, nullptr, X, C, T, N, K, split_k, stream, b);
}

SKGEMM_API int skgemm_mxfp4_batched(const void* Wq, const void* Wscale, const void* X, void* C,
                                    int T, int N, int K, int split_k, int L, size_t wq_stride,
                                    size_t wscale_stride, size_t x_stride, size_t c_stride,
                                    hipStream_t stream) {
  Batch b;
  b.L = L;
  b.bw = wq_stride;
  b.bws = wscale_stride;
  b.bx = x_stride;
  b.bc = c_stride;
  return run_gemm(skg::kMxfp4, Wq, Wscale, X, C, T, N, K, split_k, stream, b);
}

SKGEMM_API int skgemm_mxfp8_batched(const void* Wq8, const void* Wscale, const void* X, void* C,
                                    int T, int N, int K, int split_k, int L, size_t wq8_stride,
                                    size_t wscale_stride, size_t x_stride, size_t c_stride,
                                    hipStream_t stream) {
  Batch b;
  b.L = L;
  b.bw = wq8_stride;
  b.bws = wscale_stride;
  b.bx = x_stride;
  b.bc = c_stride;
  return run_gemm(skg::kMxfp8, Wq8, Wscale, X, C, T, N, K, split_k, stream, b);
}

SKGEMM_API int skgemm_reserve(int max_T, int max_N, int max_split_k, hipStream_t stream) {
  return skgemm_reserve_batched(max_T, max_N, max_split_k, 1, stream);
}

SKGEMM_API int skgemm_reserve_batched(int max_T, int max_N, int max_split_k, int max_L,
                                      hipStream_t stream) {
  if (max_T < 0 || max_N < 0 || max_split_k < 1 || max_split_k > 8) return SKGEMM_EINVAL;
  if (max_L < 1 || max_L > SKGEMM_MAX_BATCH) return SKGEMM_EINVAL;
  if (max_N > SKGEMM_MAX_N) return SKGEMM_ESHAPE;
  Workspace w;
  return ensure_workspace(stream, part_bytes_for(max_T, max_N, max_split_k) * (size_t)max_L,
                          counters_for(max_N) * (size_t)max_L, &w);
}

SKGEMM_API int skgemm_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int rc = SKGEMM_OK;
  // Each workspace is freed with its own device current; the caller's
  // current device is restored afterwards.
  int caller_dev = -1;
  if (hipGetDevice(&caller_dev) != hipSuccess) caller_dev = -1;
  std::vector<std::pair<int, Workspace>> all(g_retired.begin(), g_retired.end());
  for (auto& kv : g_ws) all.emplace_back(kv.first.first, kv.second);
  for (auto& dw : all) {
    hipError_t e = hipSetDevice(dw.first);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = hip_fail(e);
    if (dw.second.part) (void)hipFree(dw.second.part);
    if (dw.second.cnt) (void)hipFree(dw.second.cnt);
  }
  g_ws.clear();
  g_retired.clear();
  if (caller_dev >= 0) {
    const hipError_t e = hipSetDevice(caller_dev);
    if (e != hipSuccess && rc == SKGEMM_OK) rc = hip_fail(e);
  }
  return rc;
}

SKGEMM_API int skgemm_mxfp4_dequant(const void* Wq, const void* Wscale, void* W_out, int N, int K,
                                    hipStream_t stream) {
  if (N < 0 || K < 0) return SKGEMM_EINVAL;
  if (K % 32 != 0) return SKGEMM_ESHAPE;
  if (N == 0 || K == 0) return SKGEMM_OK;
  if (!Wq || !Wscale || !W_out) return SKGEMM_EINVAL;
  if (!aligned16(Wq) || !aligned16(W_out)) return SKGEMM_EALIGN;
  hipError_t e = skg::launch_mxfp4_dequant(Wq, Wscale, W_out, N, K, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_mxfp8_dequant(const void* Wq8, const void* Wscale, void* W_out, int N, int K,
                                    hipStream_t stream) {
  if (N < 0 || K < 0) return SKGEMM_EINVAL;
  if (K % 32 != 0) return SKGEMM_ESHAPE;
  if (N == 0 || K == 0) return SKGEMM_OK;
  if (!Wq8 || !Wscale || !W_out) return SKGEMM_EINVAL;
  if (!aligned16(Wq8) || !aligned16(W_out)) return SKGEMM_EALIGN;
  hipError_t e = skg::launch_mxfp8_dequant(Wq8, Wscale, W_out, N, K, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_pack_bf16(const float* in, uint32_t* out, size_t n_pairs, hipStream_t stream) {
  if (n_pairs == 0) return SKGEMM_OK;
  if (!in || !out) return SKGEMM_EINVAL;
  if (!aligned16(in) || !aligned16(out)) return SKGEMM_EALIGN;
  hipError_t e = skg::launch_pack_bf16(in, out, n_pairs, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_pack_e4m3(const float* in, uint32_t* out, size_t n_quads, hipStream_t stream) {
  if (n_quads == 0) return SKGEMM_OK;
  if (!in || !out) return SKGEMM_EINVAL;
  if (!aligned16(in) || !aligned16(out)) return SKGEMM_EALIGN;
  hipError_t e = skg::launch_pack_e4m3(in, out, n_quads, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_wave_sum(const float* in, float* out, size_t n_waves, hipStream_t stream) {
  if (n_waves == 0) return SKGEMM_OK;
  if (!in || !out) return SKGEMM_EINVAL;
  if (!aligned16(in) || !aligned16(out)) return SKGEMM_EALIGN;
  hipError_t e = skg::launch_wave_sum(in, out, n_waves, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_tactic_for(int T, int N, int K, int split_k, int weight_format, char* buf,
                                 size_t buf_len) {
  if (weight_format < skg::kBf16 || weight_format > skg::kMxfp8) return SKGEMM_EINVAL;
  int rc = check_gemm(weight_format, nullptr, nullptr, nullptr, nullptr, T, N, K, split_k, false);
  if (rc != SKGEMM_OK) return rc;
  skg::Tactic t{};
  const int tb = std::min(std::max(T, 1), kTokenBlock);
  if (!skg::pick_tactic(tb, N, K, split_k, weight_format, &t)) return SKGEMM_ESHAPE;
  const int blocks = (T + kTokenBlock - 1) / kTokenBlock;
  if (buf != nullptr && buf_len > 0) {
    snprintf(buf, buf_len,
             "{\"nt\": %d, \"rg\": %d, \"wk\": %d, \"wn\": %d, \"d\": %d, \"c\": %d, \"kc\": %d, "
             "\"tile_n\": %d, \"threads\": %d, \"lds\": %d, \"grid\": %d, \"split_k\": %d, "
             "\"token_blocks\": %d, \"mxfp4\": %d, \"weight_format\": %d, \"kind\": \"%s\", "
             "\"shape\": %d, \"fold\": %d, \"pdefer\": %d, \"handoff\": \"%s\"}",
             t.nt, t.rg, t.wk, t.wn, t.d, t.c, t.kc, t.tile_n, t.threads, t.lds, t.grid, split_k,
             blocks, t.wf == skg::kMxfp4 ? 1 : 0, t.wf, t.kind == 3 ? "wide" : t.kind == 2 ? "cluster" : (t.kind == 1 ? "stream" : "tiled"), t.shape,
             t.kind == 2 ? t.fold : 1, t.pdefer,
             split_k == 1 ? "none" : t.kind == 2 ? "lds"
             : (knob(skg::kKnobHandoff, kDefaultHandoff) == 1 && skg::tactic_mailbox(t)) ? "mailbox" : "counter");
  }
  return SKGEMM_OK;
}

SKGEMM_API int skgemm_set_timeline(void* buf, size_t capacity) {
  if (buf != nullptr && ((uintptr_t)buf & 7u) != 0) return SKGEMM_EALIGN;
  g_stamps_cap.store(buf ? capacity : 0);
  g_stamps.store(static_cast<uint64_t*>(buf));
  return SKGEMM_OK;
}

SKGEMM_API int skgemm_health(uint32_t* words, size_t n_words, hipStream_t stream) {
  if (words == nullptr && n_words > 0) return SKGEMM_EINVAL;
  for (size_t i = 0; i < n_words; ++i) words[i] = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  Workspace w;
  {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find(std::make_pair(dev, stream));
    if (it == g_ws.end() || it->second.cnt == nullptr) return SKGEMM_OK;  // nothing ran yet
    w = it->second;
  }
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e);
  if (st != hipStreamCaptureStatusNone) return SKGEMM_EINVAL;
  uint32_t* health = w.cnt + w.cnt_count;
  const size_t n = std::min(n_words, (size_t)skg::kHealthWords);
  e = hipStreamSynchronize(stream);
  if (e == hipSuccess && n > 0) e = hipMemcpy(words, health, n * sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemsetAsync(health, 0, skg::kHealthWords * sizeof(uint32_t), stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0) return SKGEMM_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return SKGEMM_EALIGN;
  const hipError_t e = skg::launch_read_probe(src, bytes, sink, stream);
  return e == hipSuccess ? SKGEMM_OK : hip_fail(e);
}

SKGEMM_API int skgemm_set_override(int knob, int value) {
  if (knob < 0 || knob >= skg::kKnobCount || value < -1) return SKGEMM_EINVAL;
  g_knobs[knob].store(value + 1, std::memory_order_relaxed);
  return SKGEMM_OK;
}

SKGEMM_API const char* skgemm_strerror(int code) {
  switch (code) {
    case SKGEMM_OK: return "success";
    case SKGEMM_EINVAL: return "invalid argument (null pointer, negative size or split_k not in {1,2,4,8})";
    case SKGEMM_EALIGN: return "pointer not 16-byte aligned";
    case SKGEMM_ESHAPE: return "unsupported shape (N % 16, K % (32*split_k) or K % (128*split_k) for MXFP4, or size limit)";
    case SKGEMM_ENOMEM: return "split-K workspace could not be allocated (or must grow during stream capture: call skgemm_reserve first)";
    case SKGEMM_EHIP: return "HIP runtime error (see skgemm_last_hip_error)";
    case SKGEMM_ESCRATCH: return "the call needs more split-K partials than the fixed scratch of skgemm_bf16_noalloc holds (split_k * min(T,128) * N * 4 bytes; see SKGEMM_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown skgemm status";
}

SKGEMM_API int skgemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
