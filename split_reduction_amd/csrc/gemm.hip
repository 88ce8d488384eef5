// Split-K decode GEMM kernels for gfx950: C[T, N] = X[T, K] . W[N, K]^T.
//
// The method (page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk,
// module summary and SplitKGemm): each split rank accumulates one exact,
// contiguous K slice in FP32 (SplitKGemm.kernel: K splits evenly, rank r takes
// the r-th slice); the partials are reduced once, in rank order, cast and
// stored once (SplitKGemm.epilog_warp). The weights take the MFMA's row
// operand (swap-AB: kernel-M carries public N), so a 16-row weight tile
// meets a 16-token activation tile in each v_mfma_f32_16x16x32_bf16.
//
// MI355X design, one workgroup = (output tile of TILE_N features, split rank):
//  * Weight stream: every lane issues 16-byte buffer loads with the streaming
//    (NT) policy straight into MFMA A operands -- the role of the pages'
//    evict-first weight TMA (SplitKGemm.weight_warp, _tma_load_evict_first).
//    D load steps per row group stay in flight, all issued before any use
//    (page vllm.models.deepseek_v41.amd.mono.common.ops, batched_rounds).
//    Past the end a load takes an out-of-range offset and returns zeros
//    without a memory access (page vllm.models.muse_spark.amd.mono.kernels.dev,
//    ld_vec_if).
//  * Activations: the workgroup stages its X slice [T_pad, kc] in LDS in
//    MFMA-operand order, rows t >= T read as zeros with no memory access
//    (SplitKGemm.activation_warp's role). Each B-operand read is one
//    conflict-free 1 KiB ds_read_b128 per wave.
//  * The WK waves of a workgroup split its K slice; their FP32 accumulators
//    are summed through LDS in wave order 0..WK-1 (same ops page, row_sum).
//  * Across split ranks: each rank stores its FP32 tile to a global partial
//    buffer and bumps the tile's counter (acq_rel, agent scope). The rank that
//    arrives last sums partials 0..S-1 in rank order (its own from registers),
//    rounds to bf16 (RNE) and stores C once, then returns the counter to zero.
//    Nothing spins, so no workgroup waits for another to be resident (the
//    pages' DSMEM mailbox has no equivalent across CUs).
//  * MXFP4: each lane loads 16 bytes = 32 E2M1 codes = one whole 32-element
//    scale block of one row, and decodes them into four bf16x8 A operands in
//    registers (page vllm.models.muse_spark.amd.mono.kernels.dev, fp4x8_bf16
//    and e8m0_f32). The activations are staged with the same K permutation,
//    which leaves the contraction unchanged.

#include "device/mfma.h"
#include "device/mxfp4.h"
#include "device/pack.h"
#include "device/types.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* smem, int slot) {
  return *reinterpret_cast<const u32x4*>(smem + slot * 16);
}

__device__ __forceinline__ void lds_write16(uint8_t* smem, int slot, u32x4 v) {
  *reinterpret_cast<u32x4*>(smem + slot * 16) = v;
}

}  // namespace

template <int NT, int RG, int WK, int WN, int D, bool MX>
__global__ __launch_bounds__(64 * WK * WN) void splitk_gemm_kernel(GemmParams p) {
  constexpr int THREADS = 64 * WK * WN;
  constexpr int TILE_N = 16 * RG * WN;
  constexpr int STEP_K = MX ? 128 : 32;  // K elements of one 16-byte lane load, per row
  constexpr int SUB = MX ? 4 : 1;        // MFMA K-steps per load step
  constexpr int TPAD = 16 * NT;
  constexpr int XBATCH = 4;              // staging loads issued before their LDS writes

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wk = wave % WK;
  const int wn = wave / WK;
  const int g = lane >> 4;   // K block of this lane within an MFMA operand
  const int li = lane & 15;  // row (A) / token (B) of this lane

  const int S = p.S;
  const int T = p.T;
  const int K = p.K;
  const int N = p.N;
  const int tile = blockIdx.x / S;
  const int rank = blockIdx.x - tile * S;
  const int n0 = tile * TILE_N;
  const int kbase = rank * p.ks;

  // Weight rows of this tile (byte bounds below 2^31, checked on the host).
  const uint32_t wrow_bytes = MX ? (uint32_t)(K / 2) : (uint32_t)K * 2u;
  const rsrc_t wr = make_rsrc(static_cast<const uint8_t*>(p.w) + (size_t)n0 * wrow_bytes,
                              TILE_N * wrow_bytes);
  const rsrc_t sr = MX ? make_rsrc(p.wscale + (size_t)n0 * (K / 32), TILE_N * (uint32_t)(K / 32))
                       : wr;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)T * (uint32_t)K * 2u);

  uint32_t row_off[RG];
  uint32_t srow_off[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const uint32_t row = (uint32_t)((wn * RG + rg) * 16 + li);
    row_off[rg] = row * wrow_bytes;
    srow_off[rg] = row * (uint32_t)(K / 32);
  }

  f32x4 acc[RG][NT];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ring[D][RG];
  uint32_t sring[D][RG];

  for (int c = 0; c < p.nchunks; ++c) {
    const int kc0 = kbase + c * p.kc;  // first K element of the chunk
    const int cs = p.kc / STEP_K;      // load steps in the chunk
    const int n_i = (cs - wk + WK - 1) / WK;  // this wave's steps: j = wk + WK * i

    // Weight prologue: D load steps, issued before the staging below so the
    // X loads' latency hides under the weight loads'.
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const bool ok = s < n_i;
      const int kel = kc0 + (wk + WK * s) * STEP_K;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if constexpr (MX) {
          ring[s][rg] = ld16_if<kPolicyStream>(ok, wr, row_off[rg] + kel / 2 + 16 * g);
          sring[s][rg] = ld1_if<kPolicyStream>(ok, sr, srow_off[rg] + kel / 32 + g);
        } else {
          ring[s][rg] = ld16_if<kPolicyStream>(ok, wr, row_off[rg] + kel * 2 + 16 * g);
        }
      }
    }

    if (c > 0) __syncthreads();  // every wave is done reading the previous chunk

    // Stage X[0:TPAD, kc0 : kc0 + kc) into LDS in MFMA B-operand order.
    // Piece (t, q) = 8 bf16 at chunk-local K 8q of row t; consecutive threads
    // take consecutive rows, so a wave writes 1 KiB of LDS contiguously.
    {
      const int pieces = TPAD * (p.kc / 8);
      for (int p0 = tid; p0 < pieces; p0 += THREADS * XBATCH) {
        u32x4 v[XBATCH];
#pragma unroll
        for (int b = 0; b < XBATCH; ++b) {
          const int pc = p0 + b * THREADS;
          const int t = pc % TPAD;
          const int k = (pc / TPAD) * 8;
          const bool ok = (pc < pieces) && (t < T);
          v[b] = ld16_if(ok, xr, ((uint32_t)t * (uint32_t)K + (uint32_t)(kc0 + k)) * 2u);
        }
#pragma unroll
        for (int b = 0; b < XBATCH; ++b) {
          const int pc = p0 + b * THREADS;
          if (pc < pieces) {
            const int t = pc % TPAD;
            const int k = (pc / TPAD) * 8;
            int slot;
            if constexpr (MX) {
              const int m = k / 128, gg = (k % 128) / 32, d = (k % 32) / 8;
              slot = ((m * 4 + d) * NT + t / 16) * 64 + gg * 16 + (t % 16);
            } else {
              const int j = k / 32, gg = (k % 32) / 8;
              slot = (j * NT + t / 16) * 64 + gg * 16 + (t % 16);
            }
            lds_write16(smem, slot, v[b]);
          }
        }
      }
    }
    __syncthreads();

    // One load step: RG weight operands against NT activation operands.
    auto compute = [&](const u32x4 (&a)[RG], const uint32_t (&sc)[RG], int i) {
      const int j = wk + WK * i;  // chunk-local load step
#pragma unroll
      for (int sub = 0; sub < SUB; ++sub) {
        bf16x8 b[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          b[tt] = as_bf16x8(lds_read16(smem, ((j * SUB + sub) * NT + tt) * 64 + lane));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          bf16x8 af;
          if constexpr (MX) {
            af = fp4x8_bf16(a[rg][sub], e8m0_f32(sc[rg]));
          } else {
            af = as_bf16x8(a[rg]);
          }
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = mfma_bf16(af, b[tt], acc[rg][tt]);
        }
      }
    };

    int i0 = 0;
    for (; i0 + D <= n_i; i0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        u32x4 a[RG];
        uint32_t sc[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          a[rg] = ring[s][rg];
          sc[rg] = sring[s][rg];
        }
        const int inext = i0 + s + D;
        const bool ok = inext < n_i;
        const int kel = kc0 + (wk + WK * inext) * STEP_K;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          if constexpr (MX) {
            ring[s][rg] = ld16_if<kPolicyStream>(ok, wr, row_off[rg] + kel / 2 + 16 * g);
            sring[s][rg] = ld1_if<kPolicyStream>(ok, sr, srow_off[rg] + kel / 32 + g);
          } else {
            ring[s][rg] = ld16_if<kPolicyStream>(ok, wr, row_off[rg] + kel * 2 + 16 * g);
          }
        }
        compute(a, sc, i0 + s);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (i0 + s < n_i) compute(ring[s], sring[s], i0 + s);
    }
  }

  // ---- reduction over the WK waves, in wave order, through LDS ----------
  // Waves wk >= 1 park their accumulators in LDS; wave wk = 0 of each N
  // column adds them to its own in wave order 1..WK-1, so every output is
  // ((a0 + a1) + a2) + ... as in the pages' row_sum. Wave 0 of each column
  // then owns the tile's quads: lane l holds tokens tt*16 + l%16 of features
  // (wn*RG + rg)*16 + 4*(l/16) + 0..3.
  __syncthreads();  // the X region is reused
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  constexpr int QW = RG * NT * 64;  // quads of one N column of waves
  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          red[((wk - 1) * WN + wn) * QW + (rg * NT + tt) * 64 + lane] = acc[rg][tt];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            acc[rg][tt] += red[((w - 1) * WN + wn) * QW + (rg * NT + tt) * 64 + lane];
    }
  }

  const bool owner = (wk == 0);
  const int n_lane = n0 + wn * RG * 16 + 4 * g;  // feature of quad element 0, rg = 0
  const rsrc_t cr = make_rsrc(p.c, (uint32_t)T * (uint32_t)N * 2u);
  auto c_off = [&](int rg, int tt) -> uint32_t {
    return ((uint32_t)(tt * 16 + li) * (uint32_t)N + (uint32_t)(n_lane + rg * 16)) * 2u;
  };
  auto in_t = [&](int tt) -> bool { return owner && (tt * 16 + li < T); };

  if (S == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) st8_if(in_t(tt), bf16_quad(acc[rg][tt]), cr, c_off(rg, tt));
    return;
  }

  // ---- split-K hand-off across workgroups --------------------------------
  const rsrc_t pr = make_rsrc(p.part, (uint32_t)S * (uint32_t)T * (uint32_t)N * 4u);
  auto p_off = [&](int r, int rg, int tt) -> uint32_t {
    return (((uint32_t)r * (uint32_t)T + (uint32_t)(tt * 16 + li)) * (uint32_t)N +
            (uint32_t)(n_lane + rg * 16)) * 4u;
  };
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      st16_if(in_t(tt), __builtin_bit_cast(u32x4, acc[rg][tt]), pr, p_off(rank, rg, tt));
  // Every wave releases its own partial stores at agent scope before the
  // workgroup barrier; thread 0's arrival then carries them to the last rank.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (old == (uint32_t)(S - 1));
    if (last) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0 || !owner) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // The last rank to arrive sums the ranks' partials in rank order 0..S-1,
  // taking its own from registers, rounds once and stores C once.
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const bool ok = in_t(tt);
      f32x4 tot = (rank == 0) ? acc[rg][tt]
                              : __builtin_bit_cast(f32x4, ld16_if(ok, pr, p_off(0, rg, tt)));
      for (int r = 1; r < S; ++r) {
        const f32x4 v = (r == rank) ? acc[rg][tt]
                                    : __builtin_bit_cast(f32x4, ld16_if(ok, pr, p_off(r, rg, tt)));
        tot += v;
      }
      st8_if(ok, bf16_quad(tot), cr, c_off(rg, tt));
    }
  }
}

// ---------------------------------------------------------------------------
// configurations and dispatch
// ---------------------------------------------------------------------------

namespace {

struct Shape {
  int rg, wk, wn, d;
};

// The instantiated workgroup shapes (per NT and weight format).
constexpr Shape kShapes[] = {
    {1, 4, 1, 8},  // tile_n 16: many small tiles for small N * split_k
    {2, 4, 1, 8},  // tile_n 32
    {4, 4, 1, 4},  // tile_n 64
    {2, 2, 2, 4},  // tile_n 64, two waves share each staged X chunk
};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

constexpr int kMaxXLds = 56 * 1024;  // LDS for the staged X chunk
constexpr int kMaxLds = 60 * 1024;   // dynamic LDS per workgroup

template <int NT, int SH, bool MX>
hipError_t launch_one(const Tactic& t, const GemmParams& p, hipStream_t s) {
  constexpr Shape sh = kShapes[SH];
  auto kern = splitk_gemm_kernel<NT, sh.rg, sh.wk, sh.wn, sh.d, MX>;
  hipLaunchKernelGGL(kern, dim3(t.grid), dim3(t.threads), t.lds, s, p);
  return hipGetLastError();
}

template <int NT, bool MX>
hipError_t launch_nt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (sh) {
    case 0: return launch_one<NT, 0, MX>(t, p, s);
    case 1: return launch_one<NT, 1, MX>(t, p, s);
    case 2: return launch_one<NT, 2, MX>(t, p, s);
    case 3: return launch_one<NT, 3, MX>(t, p, s);
  }
  return hipErrorInvalidValue;
}

template <bool MX>
hipError_t launch_fmt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.nt) {
    case 1: return launch_nt<1, MX>(sh, t, p, s);
    case 2: return launch_nt<2, MX>(sh, t, p, s);
    case 3: return launch_nt<3, MX>(sh, t, p, s);
    case 4: return launch_nt<4, MX>(sh, t, p, s);
    case 5: return launch_nt<5, MX>(sh, t, p, s);
    case 6: return launch_nt<6, MX>(sh, t, p, s);
    case 7: return launch_nt<7, MX>(sh, t, p, s);
    case 8: return launch_nt<8, MX>(sh, t, p, s);
  }
  return hipErrorInvalidValue;
}

int shape_index(const Tactic& t) {
  for (int i = 0; i < kNumShapes; ++i)
    if (kShapes[i].rg == t.rg && kShapes[i].wk == t.wk && kShapes[i].wn == t.wn &&
        kShapes[i].d == t.d)
      return i;
  return -1;
}

// Largest chunk kc that divides ks, is a multiple of `step` and whose staged
// X tile (tpad rows of bf16) fits in the LDS budget.
int pick_kc(int ks, int step, int tpad) {
  if (ks == 0) return 0;
  const int units = ks / step;
  for (int m = 1; m <= units; ++m) {
    if (units % m) continue;
    const int kc = ks / m;
    if ((long)tpad * kc * 2 <= kMaxXLds) return kc;
  }
  return -1;
}

}  // namespace

bool pick_tactic(int T, int N, int K, int S, bool mx, Tactic* out) {
  Tactic t{};
  t.nt = (T + 15) / 16;
  if (t.nt < 1) t.nt = 1;
  if (t.nt > 8) return false;
  t.mx = mx ? 1 : 0;
  const int step = mx ? 128 : 32;
  const int ks = K / S;

  // Shape choice: in order of preference (larger tiles re-read X less), the
  // first whose tile divides N and that gives at least two workgroups per CU
  // (256 CUs); failing that, the one giving the most workgroups.
  static const int order_small_t[] = {2, 1, 0};
  static const int order_large_t[] = {3, 2, 1, 0};
  const int* order = (t.nt >= 4) ? order_large_t : order_small_t;
  const int norder = (t.nt >= 4) ? 4 : 3;
  int chosen = -1;
  long best_wgs = -1;
  int chosen_kc = -1, chosen_lds = 0;
  const int tpad = 16 * t.nt;
  for (int oi = 0; oi < norder; ++oi) {
    const Shape& c = kShapes[order[oi]];
    const int tile_n = 16 * c.rg * c.wn;
    if (N % tile_n) continue;
    const int kc = pick_kc(ks, step, tpad);
    if (kc < 0) continue;
    const int x_lds = tpad * kc * 2;
    const int red_lds = (c.wk - 1) * c.wn * c.rg * t.nt * 64 * 16;
    const int lds = x_lds > red_lds ? x_lds : red_lds;
    if (lds > kMaxLds) continue;
    const long wgs = (long)(N / tile_n) * S;
    if (wgs >= 512 || wgs > best_wgs) {
      best_wgs = wgs;
      chosen = order[oi];
      chosen_kc = kc;
      chosen_lds = lds;
    }
    if (wgs >= 512) break;
  }
  if (chosen < 0) return false;
  const Shape& sh = kShapes[chosen];
  t.rg = sh.rg;
  t.wk = sh.wk;
  t.wn = sh.wn;
  t.d = sh.d;
  t.tile_n = 16 * sh.rg * sh.wn;
  t.threads = 64 * sh.wk * sh.wn;
  t.kc = chosen_kc;
  t.lds = chosen_lds;
  t.grid = (N / t.tile_n) * S;
  *out = t;
  return true;
}

hipError_t launch_gemm(const Tactic& t, const GemmParams& p, hipStream_t s) {
  const int sh = shape_index(t);
  if (sh < 0) return hipErrorInvalidValue;
  return t.mx ? launch_fmt<true>(sh, t, p, s) : launch_fmt<false>(sh, t, p, s);
}

}  // namespace skg
