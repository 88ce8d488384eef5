// A chain of split-K GEMMs in one persistent launch: step i computes
// C_i[T, d_(i+1)] = A_i[T, d_i] . W_i[d_(i+1), d_i]^T with A_0 = X and
// A_i = C_(i-1), each step by the method of the other kernels (page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk, module
// summary and SplitKGemm: S contiguous K slices accumulated in FP32, summed
// once in rank order, rounded to bf16 and stored once).
//
// The launch overlap the pages get from programmatic dependent launch
// (SplitKGemm.__call__ launches with use_pdl; weight_warp issues its weight
// loads before the wait on the preceding grid and activation_warp loads the
// activations only after it) is made here inside one launch: a workgroup that
// has finished its part of step i issues the weight loads of its first tile
// of step i+1 (weights do not depend on step i), then waits at a grid-wide
// barrier until every workgroup has stored its part of C_i, and only then
// loads its activations, which are C_i. Between tiles of one step the next
// tile's weights likewise go out before the current tile's reduction.
//
// Each tile is computed as in the all-ranks-in-one-workgroup kernel: the
// workgroup's eight waves form S rank groups, rank group r streams K slice r
// of R = 16/F weight rows (K folded F ways into the MFMA operand for T <=
// 16/F tokens), the rank partials meet in LDS and are summed in rank order.
// The workgroups are launched cooperatively (all resident at once: the barrier
// waits only for running workgroups); the barrier wait is still bounded and a
// time-out is recorded in the stream's health words instead of hanging.
//
// Visibility across the XCDs' caches: C stores are device-coherent (written
// through to the level all XCDs share) and complete before a workgroup
// arrives at the barrier; the activation loads after the barrier are
// device-coherent as well, so they never hit a stale copy and need no cache
// invalidate (measured: a 32-step decode chain 12.7 -> 11.3 us a step against
// an agent-scope acquire fence after every barrier).

#include "device/mfma.h"
#include "device/out.h"
#include "device/pack.h"
#include "device/types.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

constexpr int kChainWaves = 8;
// Load steps in flight per wave (4 KiB of weights at a fold of 2). Measured
// on the T=8 K=7168 / K=2048 decode chain, per step of a 32-step chain, one
// box: 2 steps 14.7 us, 3 steps 13.1 us, 4 steps 12.8 us, 8 steps 13.9 us;
// 16 steps were slower still.
constexpr int kChainDepth = 4;

// s_waitcnt vmcnt(n) for n < 64 (expcnt and lgkmcnt left at their maxima;
// the count's low four bits sit in bits 3:0 of the immediate, its high two
// in bits 15:14): waits for all but the n youngest vector memory operations
// of this wave.
template <int N>
__device__ __forceinline__ void wait_vmem_older_than() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  handoff_order();
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
  handoff_order();
}

}  // namespace

template <int S>
__global__ __launch_bounds__(64 * kChainWaves) void splitk_chain_kernel(ChainParams p) {
  constexpr int WT = kChainWaves;
  constexpr int D = kChainDepth;
  constexpr int WR = WT / S;  // waves per rank group

  __shared__ f32x4 red[WT * 64];          // every wave's accumulators
  __shared__ float part[8 * 16 * 16];     // rank partials [rank][token][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int T = p.T;
  const int rank = wave / WR;
  const int sub = wave - rank * WR;
  const int G = gridDim.x;

  // A unit of work: tile `tile` of step `step`. Each step has its own fold
  // F (p.fold[step]): R = 16 / F weight rows per tile, STEP_K = 32 F K
  // elements per load step, one 16-byte piece per lane.
  struct Unit {
    bool ok;
    int step, tile, F, R, K, N, n_i, kbase, rot;
    rsrc_t wr, xr;
  };
  auto tiles_of = [&](int step) { return p.dims[step + 1] * p.fold[step] / 16; };
  auto make_unit = [&](int step, int tile) -> Unit {
    Unit u;
    u.step = step;
    u.tile = tile;
    u.ok = step < p.L && tile < tiles_of(step);
    const int st = u.ok ? step : 0;
    u.F = p.fold[st];
    u.R = 16 / u.F;
    u.K = p.dims[st];
    u.N = p.dims[st + 1];
    const int ks = u.K / S;
    const int cs = ks / (32 * u.F);
    u.n_i = u.ok ? (cs - sub + WR - 1) / WR : 0;
    u.kbase = rank * ks;
    // Workgroups side by side on one XCD start at different steps of the
    // slice, so they do not ask for the same activation lines at once.
    u.rot = u.n_i > 0 ? (tile >> 3) % u.n_i : 0;
    const uint32_t wrow = 2u * (uint32_t)u.K;
    u.wr = make_rsrc(static_cast<const uint8_t*>(p.w[st]) + (size_t)(u.ok ? tile : 0) * u.R * wrow,
                     (uint32_t)u.R * wrow);
    u.xr = make_rsrc(st == 0 ? p.x : p.c[st - 1], (uint32_t)T * (uint32_t)u.K * 2u);
    return u;
  };
  // The first tile of this workgroup at or after `tile` in `step`, or the
  // first of a later step that has one.
  auto next_unit = [&](int step, int tile) -> Unit {
    while (step < p.L && tile >= tiles_of(step)) {
      ++step;
      tile = blockIdx.x;
    }
    return make_unit(step, tile);
  };

  // Operand layout per fold (as in the all-ranks kernel, one piece per
  // lane): A lane (li, g) holds row li % R of fold li / R, K block g of the
  // fold's window; activation loads read contiguous runs (lane m: token
  // m / 4F, chunk m % 4F) and ds_bpermute moves them to operand lane (li, g).
  u32x4 wa[D];
  u32x4 xb[D];
  auto k_of = [&](const Unit& u, int i) -> int {
    int ir = i + u.rot;
    if (ir >= u.n_i) ir -= u.n_i;
    return u.kbase + (sub + WR * ir) * 32 * u.F;
  };
  auto issue_w = [&](const Unit& u, int slot, int i) {
    const bool ok = i < u.n_i;
    const int fa = li / u.R;
    const uint32_t a_row = (uint32_t)(li % u.R) * 2u * (uint32_t)u.K;
    const uint32_t off = a_row + (uint32_t)(k_of(u, i) + (fa * 4 + g) * 8) * 2u;
    // Folded tiles read whole 128-byte lines: the non-temporal hint.
    wa[slot] = u.F >= 2 ? ld16_if<kPolicyStream>(ok, u.wr, off) : ld16_if(ok, u.wr, off);
  };
  auto issue_x = [&](const Unit& u, int slot, int i) {
    const int xt = lane / (4 * u.F);
    const bool ok = i < u.n_i && xt < T;
    const uint32_t b_row = (uint32_t)(xt < T ? xt : 0) * (uint32_t)u.K * 2u;
    xb[slot] = ld16_if<kPolicyDeviceCoherent>(ok, u.xr, b_row + (uint32_t)(k_of(u, i) + (lane % (4 * u.F)) * 8) * 2u);
  };
  auto x_operand = [&](const Unit& u, u32x4 v) -> bf16x8 {
    const int TF = 16 / u.F;
    const int b_src = 4 * ((li % TF) * 4 * u.F + (li / TF) * 4 + g);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(b_src, (int)v[e]);
    return as_bf16x8(v);
  };

  // Grid barrier between steps, run by wave 0 (which issues no weight
  // prefetch, so that waiting for the barrier's own atomics waits for
  // nothing else). Two levels, so that no counter line takes more than a
  // few dozen device-scope atomics (those on one line are served one at a
  // time): the workgroups with the same block index mod 8 count on their
  // group's line, the last of each group on the global line, and the last
  // group moves the generation word on, which every workgroup polls. The
  // counts are never reset: every barrier adds exactly the group's size to
  // a group count and the number of groups to the global count, so the last
  // arrival is the one whose old value is one short of a multiple (the
  // group sizes divide 2^32 for power-of-two grids, and a wrap needs 2^32
  // arrivals otherwise). The generation each barrier waits for is kept per
  // workgroup: read once at the start (no barrier completes before this
  // workgroup arrives), then one more per barrier passed. Each saves a round
  // trip on the chain of dependent accesses a barrier is.
  uint32_t* const bar_gen = p.sync;
  uint32_t* const bar_glob = p.sync + kCntStride;
  const int grp = blockIdx.x & 7;
  uint32_t* const bar_grp = p.sync + (2 + grp) * kCntStride;
  const uint32_t n_grp = (uint32_t)(G < 8 ? G : 8);
  const uint32_t grp_size = (uint32_t)((G - grp + 7) / 8);
  uint32_t gen = 0;
  if (wave == 0 && lane == 0) {
    gen = __hip_atomic_load(bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmem_all();  // read before this workgroup's first arrival
  }
  auto grid_barrier = [&](int step) {
    if (wave == 0) {
      wait_vmem_all();  // this wave's C stores are complete (device-coherent)
      if (lane == 0) {
        const uint32_t target = gen + 1u;
        bool last = false;
        const uint32_t old = __hip_atomic_fetch_add(bar_grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old % grp_size == grp_size - 1) {
          const uint32_t o2 = __hip_atomic_fetch_add(bar_glob, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = o2 % n_grp == n_grp - 1;
        }
        if (last) {
          __hip_atomic_store(bar_gen, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.wait_ticks;
          while (__hip_atomic_load(bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
            if (__builtin_amdgcn_s_memrealtime() > deadline) {
              note_timeout(p.health, 0xFFFFFFFFu, (uint32_t)step, p.wait_ticks);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        gen = target;
      }
      // No activation load of the next step moves above the barrier (they
      // are device-coherent: no stale copy to drop).
      handoff_order();
    }
    __syncthreads();
  };

  // One tile's reduction: folds, waves, then ranks in order; one bf16 store
  // per row pair (device-coherent: the next step reads it on other CUs).
  // Compile-time bounds (no loop whose trip count the compiler cannot see),
  // so the wait counts before the stores leave prefetched weights in flight.
  auto reduce_store = [&]<int F>(const Unit& u, f32x4 acc) {
    constexpr int R = 16 / F;
    constexpr int TF = 16 / F;
    constexpr int PAIRS = R / 2;
    red[wave * 64 + lane] = acc;
    __syncthreads();
    const float* redf = reinterpret_cast<const float*>(red);
    const int per_rank = PAIRS * T;  // <= PAIRS * TF: T <= 16 / F
#pragma unroll
    for (int h = 0; h < (S * PAIRS * TF + 64 * WT - 1) / (64 * WT); ++h) {
      const int o = tid + h * 64 * WT;
      if (o < S * per_rank) {
        const int rk = o / per_rank;
        const int rem = o - rk * per_rank;
        const int t = rem / PAIRS;
        const int r = (rem - t * PAIRS) * 2;
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < WR; ++s2) {
          const float* wbase = redf + (size_t)((rk * WR + s2) * 64) * 4;
#pragma unroll
          for (int f = 0; f < F; ++f) {
            const int row = f * R + r;
            const int col = f * TF + t;
            const float* e = wbase + (16 * (row >> 2) + col) * 4 + (row & 3);
            v0 += e[0];
            v1 += e[1];
          }
        }
        part[(rk * 16 + t) * 16 + r] = v0;
        part[(rk * 16 + t) * 16 + r + 1] = v1;
      }
    }
    __syncthreads();
    COut co;
    co.e4m3 = false;
    co.scale = 1.0f;
    co.r = make_rsrc(p.c[u.step], (uint32_t)T * (uint32_t)u.N * 2u);
    const int n0 = u.tile * R;
    if (tid < per_rank) {
      const int t = tid / PAIRS;
      const int r = (tid - t * PAIRS) * 2;
      float v0 = part[t * 16 + r];
      float v1 = part[t * 16 + r + 1];
#pragma unroll
      for (int rk = 1; rk < S; ++rk) {
        v0 += part[(rk * 16 + t) * 16 + r];
        v1 += part[(rk * 16 + t) * 16 + r + 1];
      }
      store_pair<kPolicyDeviceCoherent>(co, true, v0, v1, (uint32_t)t * (uint32_t)u.N + (uint32_t)(n0 + r));
    }
  };

  // Barrier b separates steps b and b + 1: every workgroup passes barriers
  // 0 .. L-2 exactly once each, in order, whether or not it has tiles in a
  // step. done_step is the last barrier passed.
  int done_step = -1;
  Unit cur = next_unit(0, blockIdx.x);
  if (cur.ok) {
#pragma unroll
    for (int s = 0; s < D; ++s) issue_w(cur, s, s);
    // A first tile in a later step: its activations exist only after the
    // barriers of the steps before it.
    while (done_step + 1 < cur.step) {
      grid_barrier(done_step + 1);
      ++done_step;
    }
#pragma unroll
    for (int s = 0; s < D; ++s) issue_x(cur, s, s);
  }
  while (cur.ok) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    int q = 0;
    for (; q + D <= cur.n_i; q += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        acc = mfma_bf16(as_bf16x8(wa[s]), x_operand(cur, xb[s]), acc);
        issue_w(cur, s, q + D + s);
        issue_x(cur, s, q + D + s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s)
      if (q + s < cur.n_i) acc = mfma_bf16(as_bf16x8(wa[s]), x_operand(cur, xb[s]), acc);

    const Unit nxt = next_unit(cur.step, cur.tile + G);
    const bool same_step = nxt.ok && nxt.step == cur.step;
    // Within a step the next tile's weights go out before this tile's
    // reduction; across a step they go out after its C stores (below).
    if (same_step) {
#pragma unroll
      for (int s = 0; s < D; ++s) issue_w(nxt, s, s);
    }
    if (cur.F == 2) {
      reduce_store.template operator()<2>(cur, acc);
    } else {
      reduce_store.template operator()<1>(cur, acc);
    }

    if (!same_step) {
      // End of this workgroup's part of the step: the next step's weights go
      // out now (waves 1..7; wave 0 runs the barrier), the C stores issued
      // before them complete, and then the barrier.
      if (wave != 0) {
        if (nxt.ok) {
#pragma unroll
          for (int s = 0; s < D; ++s) issue_w(nxt, s, s);
          wait_vmem_older_than<D>();  // the older C stores, not the weights
        } else {
          wait_vmem_all();  // no weights follow: all of this wave's stores
        }
      }
      __syncthreads();  // every wave's stores complete before wave 0 arrives
      const int last = nxt.ok ? nxt.step : p.L - 1;  // barriers up to last - 1
      while (done_step + 1 < last) {
        grid_barrier(done_step + 1);
        ++done_step;
      }
      if (nxt.ok && wave == 0) {
#pragma unroll
        for (int s = 0; s < D; ++s) issue_w(nxt, s, s);
      }
    }
    if (nxt.ok) {
#pragma unroll
      for (int s = 0; s < D; ++s) issue_x(nxt, s, s);
    }
    cur = nxt;
  }
  // A workgroup with no tile left still takes part in the remaining barriers
  // (a workgroup that had no tile at all takes part in every one).
  while (done_step + 1 < p.L - 1) {
    grid_barrier(done_step + 1);
    ++done_step;
  }
}

namespace {

template <int S>
hipError_t launch_chain_s(const ChainParams& p, int grid, hipStream_t s) {
  void* args[] = {const_cast<ChainParams*>(&p)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&splitk_chain_kernel<S>), dim3(grid),
                                    dim3(64 * kChainWaves), args, 0, s);
}

}  // namespace

hipError_t launch_chain(const ChainParams& p, int grid, hipStream_t s) {
  switch (p.S) {
    case 1: return launch_chain_s<1>(p, grid, s);
    case 2: return launch_chain_s<2>(p, grid, s);
    case 4: return launch_chain_s<4>(p, grid, s);
    case 8: return launch_chain_s<8>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skg
