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
//  * Weight stream: every lane issues 16-byte buffer loads straight into
//    MFMA A operands -- the role of the pages' evict-first weight TMA
//    (SplitKGemm.weight_warp, _tma_load_evict_first). The persistent kernel
//    loads whole-line pairs with the non-temporal hint (the closer analogue
//    of evict-first); the one-tile-per-workgroup fallback loads operands
//    directly with the default policy.
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
#include "device/out.h"
#include "device/pack.h"
#include "device/types.h"
#include "device/wfmt.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

// Workgroups of the stream kernel the grid sizing assumes resident per CU:
// two when one token tile suffices, one otherwise (the X slice of up to 32
// tokens then fills most of the LDS anyway). The kernel's register budget is
// pinned to match (waves per SIMD = resident waves / 4).
constexpr int stream_wgs_per_cu(int nt) { return nt == 1 ? 2 : 1; }
constexpr int stream_waves_per_eu(int nt, int waves) {
  return (stream_wgs_per_cu(nt) * waves + 3) / 4 > 0 ? (stream_wgs_per_cu(nt) * waves + 3) / 4 : 1;
}

// Organisations of the stream kernel's waves (template MODE).
constexpr int kStreamDeferred = 0;  // every wave streams; wave 0 also stores each tile's partial
constexpr int kStreamEpilogue = 1;  // wave 0 sums, stores and hands off each tile (pipelined)
constexpr int kStreamStorer = 2;    // wave 0 only sums and stores; deferred hand-off at the end

// Register budget: resident waves per SIMD. The storer organisation runs one
// workgroup per CU (single problems).
constexpr int stream_mode_waves_per_eu(int nt, int waves, int mode) {
  return mode == kStreamStorer ? (waves + 3) / 4 : stream_waves_per_eu(nt, waves);
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* smem, int slot) {
  return *reinterpret_cast<const u32x4*>(smem + slot * 16);
}

__device__ __forceinline__ void lds_write16(uint8_t* smem, int slot, u32x4 v) {
  *reinterpret_cast<u32x4*>(smem + slot * 16) = v;
}

}  // namespace

template <int NT, int RG, int WK, int WN, int D, int C, int WF>
__global__ __launch_bounds__(64 * WK * WN) void splitk_gemm_kernel(GemmParams p) {
  select_problem(p);
  constexpr bool MX = WF != kBf16;           // block-scaled weights
  constexpr int LK = lane_k(WF);             // K elements of one lane's 16-byte piece
  constexpr int THREADS = 64 * WK * WN;
  constexpr int TILE_N = 16 * RG * WN;
  constexpr int LOADS = MX ? 1 : C;          // 16-byte weight loads per row group per step
  constexpr int SUBS = MX ? LK / 8 : C;      // MFMA K-steps per load step
  constexpr int STEP_K = MX ? 4 * LK : 32 * C;  // K elements of one load step
  constexpr int XBATCH = 4;                  // staging loads issued before their LDS writes

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

  // Weight rows of this tile: the resource starts at the tile's first row, so
  // its span is TILE_N rows (at most 256 rows of at most 2^23 bytes: 2^31).
  const uint32_t wrow_bytes = row_bytes(WF, (uint32_t)K);
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
  // Byte offset, within a weight row, of this lane's first piece of a step
  // starting at K element kel: bf16 piece c covers K elements
  // kel + 32c + 8g .. +7 (one load instruction reads 64 contiguous bytes of
  // each row); a block-scaled lane covers kel + LK*g .. +LK-1.
  auto w_lane_off = [&](int kel) -> uint32_t { return elem_byte(WF, (uint32_t)kel) + 16u * g; };

  f32x4 acc[RG][NT];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ring[D][RG][LOADS];
  uint32_t sring[D][RG];

  // Activation operand slot of (load step j, MFMA sub-step s, lane K block
  // gg, token t) in the compact LDS tile: only real tokens are stored.
  auto x_slot = [&](int j, int s, int gg, int t) -> int { return ((j * SUBS + s) * 4 + gg) * T + t; };

  for (int c = 0; c < p.nchunks; ++c) {
    const int kc0 = kbase + c * p.kc;  // first K element of the chunk
    const int cs = p.kc / STEP_K;      // load steps in the chunk
    const int n_i = (cs - wk + WK - 1) / WK;  // this wave's steps: j = wk + WK * i

    auto issue = [&](int slot_s, int i) {
      const bool ok = i < n_i;
      const int kel = kc0 + (wk + WK * i) * STEP_K;
      const uint32_t lo = w_lane_off(kel);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) ring[slot_s][rg][l] = ld16_if(ok, wr, row_off[rg] + lo + 64 * l);
        if constexpr (MX) sring[slot_s][rg] = ld1_if(ok, sr, srow_off[rg] + (kel + LK * g) / 32);
      }
    };

    // Weight prologue first: the X staging below hides under its latency.
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s, s);

    if (c > 0) __syncthreads();  // every wave is done reading the previous chunk

    // Stage X[0:T, kc0 : kc0 + kc) in LDS. Consecutive threads take
    // consecutive 8-element pieces of one token, so every 4-lane group of a
    // load reads one contiguous run.
    {
      const int kp = p.kc / 8;  // pieces per token
      const int pieces = T * kp;
      for (int p0 = tid; p0 < pieces; p0 += THREADS * XBATCH) {
        u32x4 v[XBATCH];
#pragma unroll
        for (int b = 0; b < XBATCH; ++b) {
          const int pc = p0 + b * THREADS;
          const int t = pc / kp;
          const int k = (pc - t * kp) * 8;
          v[b] = ld16_if(pc < pieces, xr, ((uint32_t)t * (uint32_t)K + (uint32_t)(kc0 + k)) * 2u);
        }
#pragma unroll
        for (int b = 0; b < XBATCH; ++b) {
          const int pc = p0 + b * THREADS;
          if (pc < pieces) {
            const int t = pc / kp;
            const int k = (pc - t * kp) * 8;
            int j, s, gg;
            if constexpr (MX) {
              j = k / STEP_K; gg = (k % STEP_K) / LK; s = (k % LK) / 8;
            } else {
              j = k / (32 * C); s = (k % (32 * C)) / 32; gg = (k % 32) / 8;
            }
            lds_write16(smem, x_slot(j, s, gg, t), v[b]);
          }
        }
      }
    }
    __syncthreads();

    // One load step: RG weight operands per MFMA sub-step against NT
    // activation operands (zero for tokens >= T).
    auto compute = [&](const u32x4 (&a)[RG][LOADS], const uint32_t (&sc)[RG], int i) {
      const int j = wk + WK * i;  // chunk-local load step
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        bf16x8 b[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const int t = tt * 16 + li;
          const bool ok = t < T;
          const u32x4 v = lds_read16(smem, x_slot(j, s, g, ok ? t : 0));
          b[tt] = as_bf16x8(ok ? v : u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          bf16x8 af;
          if constexpr (MX) {
            af = decode_operand<WF>(a[rg][0], s, e8m0_f32(sc[rg]));
          } else {
            af = as_bf16x8(a[rg][s]);
          }
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = mfma_bf16(af, b[tt], acc[rg][tt]);
        }
      }
    };

    // Steady state: consume slot s, then refill the same registers with the
    // step D ahead, so D - 1 steps stay in flight while one is multiplied and
    // no register copies (which would wait for loads) are needed.
    int i0 = 0;
    for (; i0 + D <= n_i; i0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        compute(ring[s], sring[s], i0 + s);
        issue(s, i0 + s + D);
        __builtin_amdgcn_sched_barrier(0);
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
  const COut co = make_cout(p);
  auto c_el = [&](int rg, int tt) -> uint32_t {
    return (uint32_t)(tt * 16 + li) * (uint32_t)N + (uint32_t)(n_lane + rg * 16);
  };
  auto in_t = [&](int tt) -> bool { return owner && (tt * 16 + li < T); };

  if (S == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) store_quad(co, in_t(tt), acc[rg][tt], c_el(rg, tt));
    return;
  }

  // ---- split-K hand-off across workgroups --------------------------------
  // Partials are written with device-scope coherent stores (they bypass the
  // non-coherent caches of this XCD), each wave waits for its stores to be
  // acknowledged, and thread 0 then bumps the tile's arrival counter with a
  // device-scope atomic. The last arriver reads the other ranks' partials
  // with device-scope coherent loads. No cache-wide writeback or invalidate
  // is needed.
  // Partials tile-major [S, N/16, T, 16]: a wave's store or load of one
  // token tile of a 16-row group is 1 KiB of whole lines.
  const rsrc_t pr = make_rsrc(p.part, (uint32_t)S * (uint32_t)T * (uint32_t)N * 4u);
  const uint32_t grp0 = (uint32_t)((n_lane - 4 * g) / 16);  // this wave's first 16-row group
  auto p_off = [&](int r, int rg, int tt) -> uint32_t {
    return (((uint32_t)r * (uint32_t)(N / 16) + grp0 + (uint32_t)rg) * (uint32_t)T + (uint32_t)(tt * 16 + li)) * 64u +
           16u * (uint32_t)g;
  };
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, acc[rg][tt]), pr, p_off(rank, rg, tt));
  wait_vmem_all();
  __syncthreads();
  if (tid == 0) {
    uint32_t* const cnt = p.cnt + (size_t)tile * kCntStride;  // one 128-byte line each
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (old == (uint32_t)(S - 1));
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0 || !owner) return;
  handoff_order();  // the partial loads below stay after the arrival

  // The last rank to arrive sums the ranks' partials in rank order 0..S-1,
  // taking its own from registers, rounds once and stores C once.
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const bool ok = in_t(tt);
      f32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < S && r != rank)
          v[r] = __builtin_bit_cast(f32x4, ld16_coherent_if(ok, pr, p_off(r, rg, tt)));
      }
      f32x4 tot = (rank == 0) ? acc[rg][tt] : v[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) {
        if (r < S) tot += (r == rank) ? acc[rg][tt] : v[r];
      }
      store_quad(co, ok, tot, c_el(rg, tt));
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent streaming kernel (16-row tiles, X staged once per workgroup)
// ---------------------------------------------------------------------------
//
// grid = S * G workgroups; workgroup (gi, rank) owns K slice `rank` and stages
// that slice of X in LDS once, shared by all its waves for all its tiles.
// Weights stream through one register ring per wave that runs on across
// tile boundaries, so neither the staging nor the load latency is paid per
// tile; each ring slot is a whole-line load pair (rows 0-7 and 8-15 over two
// 64-byte windows, non-temporal), rearranged into MFMA operands at use.
// Organisations of the waves (MODE):
//
// * Deferred, WK > 1: all WK waves stream, splitting every tile's K slice
//   (interleaved load steps). At a tile's end they meet in LDS; wave 0 adds
//   the others' sums in wave order (the pages' row_sum) and stores the tile's
//   FP32 partial (device-coherent) or, without a split, the bf16 output.
// * Storer, WK > 1: as deferred, but wave 0 does not stream: waves 1..WK-1
//   park their sums and wave 0 adds them in wave order and stores. Its
//   stores then share no completion counter with a weight ring: a
//   device-coherent store is acknowledged late, and a streaming wave that
//   issued one stalls on it at its next ring wait (measured: without
//   mid-stream stores T=32 K=7168 N=18432 runs 59 instead of 65 us).
// * Epilogue, WK > 1: wave 0 is a dedicated epilogue wave (the pages'
//   SplitKGemm keeps weight, MMA and epilogue roles in separate warps) and
//   waves 1..WK-1 stream. The epilogue wave sums the parked partials in wave
//   order and runs the split-K hand-off as a per-tile pipeline: store the
//   partial, one tile later bump the tile's counter, one tile later load the
//   ranks' partials if it arrived last, one tile later sum them in rank order
//   and store C, waiting only for its own operations of the previous stage.
// * WK == 1 (deferred): each of the WN waves streams its own tiles (column
//   gi*WN + wn takes tiles gi*WN + wn, + G*WN, ...) and stores its own
//   partials.
//
// Without an epilogue wave the hand-off is deferred to the workgroup's end:
// loads and stores share one completion counter, so waiting for a store
// mid-stream would drain the ring. At the end each wave takes every WK-th
// tile: one vector atomic bumps all their counters (a lane per tile) and the
// tiles it arrived last on are finished two at a time, all partial loads in
// flight before the sums.
template <int NT, int WK, int WN, int D, int C, int MODE, int WF>
__global__ __launch_bounds__(64 * WK * WN)
__attribute__((amdgpu_waves_per_eu(stream_mode_waves_per_eu(NT, WK * WN, MODE))))
void splitk_stream_kernel(GemmParams p) {
  select_problem(p);
  constexpr bool EPI = MODE == kStreamEpilogue;
  constexpr bool STORER = MODE == kStreamStorer;
  constexpr bool SIDE = EPI || STORER;  // wave 0 is a side wave that does not stream
  constexpr bool MX = WF != kBf16;  // block-scaled weights
  constexpr int LK = lane_k(WF);     // K elements of one lane's 16-byte piece
  constexpr int THREADS = 64 * WK * WN;
  constexpr int LOADS = MX ? 1 : C;
  constexpr int SUBS = MX ? LK / 8 : C;
  constexpr int STEP_K = MX ? 4 * LK : 32 * C;
  constexpr int XBATCH = 4;
  constexpr int SWK = SIDE ? WK - 1 : WK;   // streaming waves per tile
  constexpr int PARKED = SIDE ? SWK : WK - 1;  // partial sums parked in LDS per tile
  constexpr int RED_QUADS = (PARKED > 0 ? PARKED : 1) * NT * 64;  // one parity half
  // Whole-line weight loads (rows 0-7, rows 8-15 of the tile over two 64-byte
  // windows), turned into the two windows' operands at use, with the
  // non-temporal hint. bf16 with two pieces per step: the two windows are the
  // step's pieces (LINES). One piece per step (block-scaled, or bf16 C = 1):
  // a ring slot holds two consecutive steps, one window each (PAIRS), and
  // the slot's scale bytes come in one 8- (MXFP4) or 4-byte (MXFP8) load.
  constexpr bool LINES = !MX && C == 2;
  constexpr bool PAIRS = LOADS == 1;
  constexpr int SLOT_K = PAIRS ? 2 * STEP_K : STEP_K;  // K elements of one ring slot
  constexpr int RLOADS = PAIRS ? 2 : LOADS;            // 16-byte loads per lane per slot
  constexpr int DR = PAIRS ? (D / 2 > 0 ? D / 2 : 1) : D;  // ring slots (same bytes in flight)
  constexpr int WPOL = kPolicyStream;
  static_assert(WK == 1 || WN == 1, "waves that split a tile form one column");
  static_assert(!SIDE || (WK > 1 && WN == 1), "a side wave serves one column of streaming waves");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_tag;  // mailbox tag of this launch

  // Optional phase stamps (s_memrealtime, 100 MHz): entry, X staged, stream
  // done, own partial stores complete, exit, and in the counter hand-off the
  // arrivals done and the owned tiles' polls done (wave 0's view).
  uint64_t stamp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  stamp[0] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wk = wave % WK;
  const int wn = wave / WK;
  const int g = lane >> 4;
  const int li = lane & 15;
  const bool epi_wave = SIDE && wave == 0;  // the side wave (epilogue or storer)
  // Mailbox epoch (page vllm.models.muse_spark.amd.mono.kernels.dev, module
  // note: tags are the epoch of a device word bumped once per pass, so
  // nothing is ever zeroed): read here, before this workgroup counts itself
  // as started; the last workgroup to start advances the word for the next
  // launch, when every workgroup of this one has read it.
  uint32_t epoch0 = 0;
  if (!EPI && p.mailbox && tid == 0)
    epoch0 = __hip_atomic_load(p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int sw = SIDE ? wk - 1 : wk;  // index among the streaming waves of the tile

  const int S = p.S;
  const int T = p.T;
  const int K = p.K;
  const int N = p.N;
  const int G = gridDim.x / S;
  const int gi = blockIdx.x / S;
  const int rank = blockIdx.x - gi * S;
  const int kbase = rank * p.ks;
  const int n_tiles = N / 16;
  const int col = gi * WN + wn;   // this wave column's first tile
  const int cstride = G * WN;     // distance between its tiles
  const int ntl = (col < n_tiles) ? (n_tiles - col + cstride - 1) / cstride : 0;
  const int cs = p.ks / SLOT_K;  // ring slots per tile (whole slice)
  const int n_i = epi_wave ? 0 : (cs - sw + SWK - 1) / SWK;  // this wave's slots per tile
  const int total = ntl * n_i;

  const uint32_t wrow_bytes = row_bytes(WF, (uint32_t)K);
  const rsrc_t wr = make_rsrc(p.w, (uint32_t)N * wrow_bytes);
  const rsrc_t sr = MX ? make_rsrc(p.wscale, (uint32_t)N * (uint32_t)(K / 32)) : wr;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)T * (uint32_t)K * 2u);
  const COut co = make_cout(p);
  // Partials: FP32, tile-major [S, N/16, T, 16]: rank r's partial of one
  // 16-row tile is T x 64 contiguous bytes, so a wave's store or read-back
  // of a token tile covers whole lines (with [S, T, N] it is 16 runs of 64
  // bytes, N * 4 bytes apart). In the mailbox hand-off each value is an
  // 8-byte (value, tag) pair in the same order.
  const rsrc_t pr = make_rsrc(p.part, (uint32_t)S * (uint32_t)T * (uint32_t)N * (p.mailbox ? 8u : 4u));
  // Arrival counter of a 16-row tile: one 128-byte line each, so the S
  // ranks' arrivals and the owner's polls of one tile meet no other tile's
  // (measured: 1-3 us off the hand-off tail of T=32 K=7168 N=18432).
  auto cnt_of = [&](int tile) { return p.cnt + (size_t)tile * kCntStride; };

  // X slot of (load step j, sub-step s, lane K block gg, token t): compact tile.
  // Slot of token t's 8 elements at (step j, sub-step s, lane block gg).
  // The staging writes give consecutive lanes consecutive K chunks of one
  // token, T slots apart: with T a power of two that puts 16 lanes on the
  // same banks. The token index is therefore XOR-ed with the low bits of the
  // chunk (a permutation of the tokens inside each chunk, at most 16 wide, so
  // the reads of 16 consecutive tokens stay one 256-byte block). Measured
  // with conflict-free writes: T=16 staging 3.3 -> 2.1 us, the launch 1 us
  // shorter (K=N=16384).
  const int xsw = (T & (T - 1)) == 0 ? (T < 16 ? T : 16) - 1 : 0;
  auto x_slot = [&](int j, int s, int gg, int t) -> int {
    const int base = (j * SUBS + s) * 4 + gg;
    return base * T + (t ^ (base & xsw));
  };
  f32x4* red_base = reinterpret_cast<f32x4*>(smem + (size_t)T * p.ks * 2);  // 16-byte aligned
  // With p.pdefer, tile k's FP32 partial waits in LDS (after the reduction
  // buffers) until the stream ends: NT * 64 quads per tile.
  f32x4* pbuf = red_base + (WK > 1 ? 2 * RED_QUADS : 0);

  // ---- weight ring (streaming waves) -------------------------------------
  int pf_i = 0;
  uint32_t pf_row = (uint32_t)(col * 16) * wrow_bytes + line_pair_offset(li, 0, wrow_bytes);
  uint32_t pf_srow = (uint32_t)(col * 16 + li) * (uint32_t)(K / 32);  // scales: operand layout
  const uint32_t row_step = (uint32_t)(cstride * 16) * wrow_bytes;
  const uint32_t srow_step = (uint32_t)(cstride * 16) * (uint32_t)(K / 32);
  u32x4 ring[DR][RLOADS];
  u32x2 sring[DR];
  int issued = 0;
  auto issue = [&](int slot) {
    const bool ok = issued < total;
    const int kel = kbase + (sw + SWK * pf_i) * SLOT_K;
    const uint32_t lo = elem_byte(WF, (uint32_t)kel) + 16u * g;
#pragma unroll
    for (int l = 0; l < RLOADS; ++l) ring[slot][l] = ld16_if<WPOL>(ok, wr, pf_row + lo + 8u * wrow_bytes * l);
    if constexpr (MX) {
      // The slot's 2 * STEP_K / 32 scale bytes of row li (8 for MXFP4, 4 for MXFP8).
      const uint32_t so = pf_srow + (uint32_t)(kel / 32);
      if constexpr (WF == kMxfp4) {
        sring[slot] = ld8_if(ok, sr, so);
      } else {
        sring[slot] = u32x2{ld4_if(ok, sr, so), 0u};
      }
    }
    ++issued;
    if (++pf_i == n_i) {
      pf_i = 0;
      pf_row += row_step;
      pf_srow += srow_step;
    }
  };

  // ---- stage this rank's X slice once ------------------------------------
  // The first XPRE loads per thread of the slice go out first, then the
  // weight prologue, then the slice's LDS writes. Loads complete in order for
  // the wait counter, so the writes wait only for the older activation loads
  // while the first ring slots of weights arrive behind them: the weight
  // stream no longer starts only once the slice is in LDS. (Activation loads
  // issued after the prologue would wait for the weights as well; slices of
  // more than XPRE pieces per thread stage their remainder that way.)
  // Workgroups of one rank that share an XCD stage the same slice at the same
  // time; each starts at a different point of it (a rotation of the piece
  // order) so that their requests for the same lines do not queue on one L2
  // channel together.
  // Pieces are 16-byte chunks, K fastest (piece q: token q / kp, chunk
  // q % kp), so every 4-lane group of a load reads one contiguous run.
  // Loads per thread issued ahead of the weights: with 512 lanes 128 KiB
  // (two token tiles), 64 KiB (one, one workgroup per CU), or 32 KiB where
  // two workgroups share a CU's registers.
  constexpr int XPRE = NT > 1 ? 16 : (STORER ? 8 : 4);
  const int kp = p.ks / 8;  // chunks per token
  const int pieces = T * kp;
  const int rot = (int)(((unsigned)gi % 32u) * (unsigned)(pieces / 32));
  auto piece = [&](int pc) -> int {
    const int q = pc + rot;
    return q >= pieces ? q - pieces : q;
  };
  auto stage_load = [&]<int NB>(int p0, u32x4 (&v)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int pc = p0 + b * THREADS;
      const int q = piece(pc);
      const int t = q / kp;
      const int k = (q - t * kp) * 8;
      v[b] = ld16_if(pc < pieces, xr, ((uint32_t)t * (uint32_t)K + (uint32_t)(kbase + k)) * 2u);
    }
  };
  auto stage_store = [&]<int NB>(int p0, const u32x4 (&v)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int pc = p0 + b * THREADS;
      if (pc < pieces) {
        const int q = piece(pc);
        const int t = q / kp;
        const int k = (q - t * kp) * 8;
        int j, s2, gg;
        if constexpr (MX) {
          j = k / STEP_K; gg = (k % STEP_K) / LK; s2 = (k % LK) / 8;
        } else {
          j = k / (32 * C); s2 = (k % (32 * C)) / 32; gg = (k % 32) / 8;
        }
        lds_write16(smem, x_slot(j, s2, gg, t), v[b]);
      }
    }
  };
  // With one token tile (T <= 16) the slice is small and staging short: the
  // prologue then goes out after the barrier as before (measured: issuing it
  // first gained 1-1.6 us at T=24/32 K=N=16384, and lost 0.9 us at T=1).
  constexpr bool EARLY = NT > 1;
  {
    u32x4 v[XPRE];
    stage_load(tid, v);
    __builtin_amdgcn_sched_barrier(0);  // the activation loads stay ahead of the weights
    if (EARLY && !epi_wave) {
#pragma unroll
      for (int s = 0; s < DR; ++s) issue(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    stage_store(tid, v);
    for (int p0 = tid + THREADS * XPRE; p0 < pieces; p0 += THREADS * XBATCH) {
      u32x4 w[XBATCH];
      stage_load(p0, w);
      stage_store(p0, w);
    }
  }
  if (!EPI && p.mailbox && tid == 0) s_tag = (epoch0 & 0x7FFFFFFFu) | 0x80000000u;  // never 0
  __syncthreads();
  // This workgroup counts itself as started (after reading the epoch). The
  // count comes back long before the workgroup ends, where the last to start
  // advances the epoch: nothing waits for it here (256 device-scope atomics on
  // one line are served one at a time, several microseconds in all).
  uint32_t started_old = 0;
  if (!EPI && p.mailbox && tid == 0)
    started_old = __hip_atomic_fetch_add(p.epoch + kCntStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!EARLY && !epi_wave) {
#pragma unroll
    for (int s = 0; s < DR; ++s) issue(s);
  }
  stamp[1] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

  // Thread 0 of each workgroup writes the stamps (vector stores).
  auto write_stamps = [&]() {
    if (p.stamps != nullptr && tid == 0) {
      stamp[4] = __builtin_amdgcn_s_memrealtime();
      const rsrc_t sr8 = make_rsrc(p.stamps + (size_t)blockIdx.x * 8, 64);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st8_if(true, u32x2{(uint32_t)stamp[i], (uint32_t)(stamp[i] >> 32)}, sr8, 8u * i);
    }
  };

  // C / partial offsets of this lane's quad (token tt*16 + li, features
  // tile*16 + 4g .. +3).
  auto c_el = [&](int tile, int tt) -> uint32_t {
    return (uint32_t)(tt * 16 + li) * (uint32_t)N + (uint32_t)(tile * 16 + 4 * g);
  };
  auto p_off = [&](int r, int tile, int tt) -> uint32_t {
    return (((uint32_t)r * (uint32_t)n_tiles + (uint32_t)tile) * (uint32_t)T + (uint32_t)(tt * 16 + li)) * 64u +
           16u * (uint32_t)g;
  };
  auto in_t = [&](int tt) -> bool { return tt * 16 + li < T; };

  // Mailbox slot of this lane's quad: element (r, tile, token, f) is the
  // 8-byte pair at (((r * N/16 + tile) * T + token) * 16 + f) * 8, the same
  // tile-major order as the plain partials, the quad's four pairs in two
  // 16-byte halves (page vllm.models.muse_spark.amd.mono.kernels.dev,
  // mb_put2: two (value, tag) pairs per 16-byte store; mb_poll: reload until
  // every tag matches).
  auto m_off = [&](int r, int tile, int tt) -> uint32_t {
    return (((uint32_t)r * (uint32_t)n_tiles + (uint32_t)tile) * (uint32_t)T + (uint32_t)(tt * 16 + li)) * 128u +
           32u * (uint32_t)g;
  };
  // This rank's partial of (tile, token tile tt), device-coherent: a plain
  // FP32 quad, or in the mailbox two tagged halves.
  auto put_partial = [&](int tile, int tt, f32x4 v) {
    if (p.mailbox) {
      const uint32_t tag = s_tag;
      const uint32_t o = m_off(rank, tile, tt);
      st16_coherent_if(in_t(tt), u32x4{__float_as_uint(v.x), tag, __float_as_uint(v.y), tag}, pr, o);
      st16_coherent_if(in_t(tt), u32x4{__float_as_uint(v.z), tag, __float_as_uint(v.w), tag}, pr, o + 16u);
    } else {
      st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, v), pr, p_off(rank, tile, tt));
    }
  };

  if constexpr (EPI) {
    if (epi_wave) {
      // ---- epilogue wave: wave-order sum and pipelined hand-off -----------
      int st_tile = -1;  // partial stores issued last stage
      int at_tile = -1;  // counter atomic issued last stage
      uint32_t at_old = 0;
      int ld_tile = -1;  // partial loads issued last stage
      f32x4 ld[NT][8];
      auto finish_stage = [&]() {
        wait_vmem_all();  // everything issued at the previous stage has completed
        if (ld_tile >= 0) {  // last arriver: rank-ordered sum, one bf16 store
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            f32x4 tot = ld[tt][0];
#pragma unroll
            for (int r = 1; r < 8; ++r)
              if (r < S) tot += ld[tt][r];
            store_quad(co, in_t(tt), tot, c_el(ld_tile, tt));
          }
          ld_tile = -1;
        }
        if (at_tile >= 0) {
          const uint32_t old = __builtin_amdgcn_readfirstlane(at_old);
          handoff_order();  // the partial loads stay after the arrival
          if (old == (uint32_t)(S - 1)) {
            if (lane == 0)
              __hip_atomic_store(cnt_of(at_tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
              for (int r = 0; r < 8; ++r)
                if (r < S)
                  ld[tt][r] = __builtin_bit_cast(f32x4, ld16_coherent_if(in_t(tt), pr, p_off(r, at_tile, tt)));
            ld_tile = at_tile;
          }
          at_tile = -1;
        }
        if (st_tile >= 0) {  // its partial stores are complete: signal
          if (lane == 0)
            at_old = __hip_atomic_fetch_add(cnt_of(st_tile), 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          at_tile = st_tile;
          st_tile = -1;
        }
      };
      for (int k = 0; k < ntl; ++k) {
        __syncthreads();  // tile k's partial sums are in LDS
        const int tile = col + cstride * k;
        const f32x4* red = red_base + (k & 1) * RED_QUADS;
        f32x4 acc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt] = red[tt * 64 + lane];
#pragma unroll 1
        for (int w = 1; w < SWK; ++w)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] += red[(w * NT + tt) * 64 + lane];
        if (S == 1) {
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) store_quad(co, in_t(tt), acc[tt], c_el(tile, tt));
          continue;
        }
        finish_stage();
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, acc[tt]), pr, p_off(rank, tile, tt));
        st_tile = tile;
      }
      stamp[2] = stamp[3] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
      for (int f = 0; f < 3; ++f) finish_stage();  // drain: finish the last tiles
      write_stamps();
      return;
    }
  }

  // ---- streaming waves ----------------------------------------------------
  f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slot i of this wave: windows w = 0, 1 of the line pair are load step
  // 2 * js + w (PAIRS) or piece w of load step js (LINES), js = sw + SWK * i.
  auto compute = [&](const u32x4 (&ld)[RLOADS], u32x2 sc, int i) {
    const int js = sw + SWK * i;
    u32x4 a[2];
    line_pair_to_operands(ld[0], ld[1], a[0], a[1]);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int j = PAIRS ? 2 * js + w : js;
#pragma unroll
      for (int s2 = 0; s2 < (PAIRS ? SUBS : 1); ++s2) {
        const int sx = PAIRS ? s2 : w;  // sub-step index in the X layout
        bf16x8 b[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const int t = tt * 16 + li;
          const bool ok = t < T;
          const u32x4 v = lds_read16(smem, x_slot(j, sx, g, ok ? t : 0));
          b[tt] = as_bf16x8(ok ? v : u32x4{0u, 0u, 0u, 0u});
        }
        bf16x8 af;
        if constexpr (MX) {
          // Scale byte of (window w, lane block g) within the slot's bytes.
          const int sb = (w * STEP_K + LK * g) / 32;
          const uint32_t word = sb < 4 ? sc[0] : sc[1];
          af = decode_operand<WF>(a[w], s2, e8m0_f32((word >> (8 * (sb & 3))) & 0xFFu));
        } else {
          af = as_bf16x8(a[w]);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma_bf16(af, b[tt], acc[tt]);
      }
    }
  };

  // End of one tile for a streaming wave.
  auto tile_end = [&](int k) {
    const int tile = col + cstride * k;
    f32x4* red = red_base + (k & 1) * RED_QUADS;
    bool storer = true;
    if constexpr (SIDE) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) red[(sw * NT + tt) * 64 + lane] = acc[tt];
      __syncthreads();
      storer = false;
    } else if constexpr (WK > 1) {
      if (wk > 0) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) red[((wk - 1) * NT + tt) * 64 + lane] = acc[tt];
      }
      __syncthreads();
      if (wk == 0) {
#pragma unroll 1
        for (int w = 1; w < WK; ++w)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] += red[((w - 1) * NT + tt) * 64 + lane];
      }
      storer = (wk == 0);
    }
    if (storer) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        if (S == 1)
          store_quad(co, in_t(tt), acc[tt], c_el(tile, tt));
        else if (p.pdefer)
          pbuf[(k * NT + tt) * 64 + lane] = acc[tt];
        else
          put_partial(tile, tt, acc[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  int c_k = 0, c_i = 0;  // consume position
  auto consumed = [&]() {
    if (++c_i == n_i) {
      tile_end(c_k);
      c_i = 0;
      ++c_k;
    }
  };

  int q = 0;
  for (; q + DR <= total; q += DR) {
#pragma unroll
    for (int s = 0; s < DR; ++s) {
      compute(ring[s], sring[s], c_i);
      issue(s);
      __builtin_amdgcn_sched_barrier(0);
      consumed();
    }
  }
#pragma unroll
  for (int s = 0; s < DR; ++s) {
    if (q + s < total) {
      compute(ring[s], sring[s], c_i);
      consumed();
    }
  }
  if (n_i == 0) {
    if (STORER && epi_wave) {
      // The storer wave: per tile, the streaming waves' sums in wave order,
      // then the tile's partial (or, with one rank, C) stored. It never
      // waits for its stores before the end, so their acknowledgements hold
      // up no weight load. Split partials that are not held in LDS are held
      // in this wave's registers (it has no weight ring) and stored HOLD
      // tiles at a time, in bursts rather than tile by tile.
      constexpr int HOLD = 16;
      auto tile_sum = [&](int k, f32x4 (&sum)[NT]) {
        const f32x4* red = red_base + (k & 1) * RED_QUADS;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) sum[tt] = red[tt * 64 + lane];
#pragma unroll 1
        for (int w = 1; w < SWK; ++w)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) sum[tt] += red[(w * NT + tt) * 64 + lane];
      };
      if (S > 1 && !p.pdefer) {
        for (int k0 = 0; k0 < ntl; k0 += HOLD) {
          f32x4 hold[HOLD][NT];
#pragma unroll
          for (int j = 0; j < HOLD; ++j) {
            if (k0 + j < ntl) {
              __syncthreads();  // tile k0 + j's sums are in LDS
              tile_sum(k0 + j, hold[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < HOLD; ++j) {
            if (k0 + j < ntl) {
              const int tile = col + cstride * (k0 + j);
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) put_partial(tile, tt, hold[j][tt]);
            }
          }
        }
      } else {
        for (int k = 0; k < ntl; ++k) {
          __syncthreads();  // tile k's sums are in LDS
          const int tile = col + cstride * k;
          f32x4 sum[NT];
          tile_sum(k, sum);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            if (S == 1)
              store_quad(co, in_t(tt), sum[tt], c_el(tile, tt));
            else
              pbuf[(k * NT + tt) * 64 + lane] = sum[tt];
          }
        }
      }
    } else {
      // A streaming wave with no steps (slice shorter than the wave count)
      // still takes part in every tile's barrier.
      for (int k = 0; k < ntl; ++k) tile_end(k);
    }
  }
  stamp[2] = stamp[3] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  if (EPI || S == 1) {
    write_stamps();
    return;
  }

  // ---- deferred hand-off ----------------------------------------------------
  // The k-th tile of a list has an owner rank, (k + gi) mod S, the same in
  // every rank of the group, so the reductions spread evenly over the ranks
  // (and over the XCDs, which the ranks map to). Every rank bumps the tile's
  // arrival counter once its partial stores are complete. The owner waits,
  // for a bounded time, until all S have arrived, then sums the partials in
  // rank order, stores C and clears the counter. If the wait runs out (a
  // peer that is not resident, e.g. under a concurrent kernel), the owner sets
  // the abandon bit and the last rank to arrive finishes the tile instead, so
  // the result never depends on the peers being resident.
  auto tile_at = [&](int k) { return col + cstride * k; };
  auto owner_of = [&](int k) { return (k + gi) % S; };
  constexpr uint32_t kArrivals = 0xFFu;  // arrival count bits of a counter
  constexpr uint32_t kAbandon = 0x100u;  // the owner stopped waiting
  const int k_first = ((rank - gi) % S + S) % S;  // first list position this rank owns
  const int n_own = (ntl > k_first) ? (ntl - k_first + S - 1) / S : 0;

  if (p.mailbox) {
    // ---- mailbox hand-off ---------------------------------------------------
    // Peers store tagged partials and do not wait; an owner polls the tagged
    // data itself (one round trip after the last partial lands: no counter
    // poll and no separate load of the partials), sums in rank order and
    // stores C, and only then adds its arrival. The arrival counter serves
    // the bounded wait alone: peers arrive once their stores are complete; an
    // owner whose wait runs out arrives with the abandon bit (after storing
    // its held partial); the arrival that brings the count to S resets it
    // and, after an abandon, finishes the tile if it is a peer's.
    const uint32_t tag = s_tag;
    if (p.pdefer) {
      __syncthreads();  // every tile's partial is in LDS
      for (int k = wk; k < ntl; k += WK) {
        if (owner_of(k) == rank) continue;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) put_partial(tile_at(k), tt, pbuf[(k * NT + tt) * 64 + lane]);
      }
    }
    // Polls the S partials of the tile at list position k until every tag is
    // this launch's (each lane its own quad), then sums them in rank order
    // and stores C: true; false if the deadline passes first. With `held`
    // this rank's partial comes from LDS.
    auto poll_finish = [&](int k, bool held, uint64_t deadline) -> bool {
      const int tile = tile_at(k);
      // Ranks whose data this lane still waits for, bit tt * 8 + r; a rank
      // whose tags match keeps its values and is not loaded again.
      uint32_t need = 0;
      f32x4 v[NT][8];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          v[tt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (r < S) {
            if (held && r == rank)
              v[tt][r] = pbuf[(k * NT + tt) * 64 + lane];
            else if (in_t(tt))
              need |= 1u << (tt * 8 + r);
          }
        }
      while (true) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            if (r < S) {
              const bool want = (need >> (tt * 8 + r)) & 1u;
              const uint32_t o = m_off(r, tile, tt);
              const u32x4 a = ld16_coherent_if(want, pr, o);
              const u32x4 b = ld16_coherent_if(want, pr, o + 16u);
              if (want && a[1] == tag && a[3] == tag && b[1] == tag && b[3] == tag) {
                v[tt][r] = f32x4{__uint_as_float(a[0]), __uint_as_float(a[2]), __uint_as_float(b[0]),
                                 __uint_as_float(b[2])};
                need &= ~(1u << (tt * 8 + r));
              }
            }
          }
        if (__builtin_amdgcn_ballot_w64(need != 0) == 0) {
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            f32x4 sum = v[tt][0];
#pragma unroll
            for (int r = 1; r < 8; ++r)
              if (r < S) sum += v[tt][r];
            store_quad(co, in_t(tt), sum, c_el(tile, tt));
          }
          return true;
        }
        if (__builtin_amdgcn_s_memrealtime() > deadline) return false;
        __builtin_amdgcn_s_sleep(8);
      }
    };
    // A take-over only starts once every partial is complete, so its poll
    // succeeds at once; it is still bounded (a record if it ever ran out).
    constexpr uint64_t kTakeoverTicks = 1000000;  // 10 ms
    auto take_over = [&](int k) {
      handoff_order();
      if (!poll_finish(k, false, __builtin_amdgcn_s_memrealtime() + kTakeoverTicks) && lane == 0)
        note_timeout(p.health, (uint32_t)tile_at(k), 0xFFFFu, (uint32_t)kTakeoverTicks);
    };

    int k0 = 0, kstep = 1;
    if constexpr (WK > 1) {
      k0 = wk;
      kstep = WK;
    }
    // Owned tiles first (their partials from the peers are, or will be,
    // stored already): k = k_first + S*m, m spread over the waves.
    const int my_own = (n_own > k0) ? (n_own - k0 + kstep - 1) / kstep : 0;
    for (int i = 0; i < my_own; ++i) {
      const int k = k_first + S * (k0 + kstep * i);
      uint32_t* const cnt = cnt_of(tile_at(k));
      const bool done = poll_finish(k, p.pdefer != 0, __builtin_amdgcn_s_memrealtime() + p.owner_wait);
      uint32_t old = 0;
      if (done) {
        if (lane == 0) {
          old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((old & kArrivals) == (uint32_t)(S - 1))
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        continue;
      }
      if (p.pdefer) {
        // The tile may go to a peer now: this rank's partial, held in LDS
        // so far, is stored and complete before the abandon.
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) put_partial(tile_at(k), tt, pbuf[(k * NT + tt) * 64 + lane]);
        wait_vmem_all();
      }
      if (lane == 0) {
        old = __hip_atomic_fetch_add(cnt, 1u + kAbandon, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (p.owner_wait > 0) note_timeout(p.health, (uint32_t)tile_at(k), (uint32_t)rank, p.owner_wait);
      }
      old = __builtin_amdgcn_readfirstlane(old);
      if ((old & kArrivals) == (uint32_t)(S - 1)) {
        // Every peer had arrived: their partials are complete. Still ours.
        if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        handoff_order();
        if (!poll_finish(k, p.pdefer != 0, __builtin_amdgcn_s_memrealtime() + kTakeoverTicks) && lane == 0)
          note_timeout(p.health, (uint32_t)tile_at(k), 0xFFFFu, (uint32_t)kTakeoverTicks);
      }
    }
    // Peer arrivals, once every wave's partial stores are complete: this
    // wave's share of the list, a lane per tile, tiles this rank owns left
    // out (their owner arrives itself).
    wait_vmem_all();
    if constexpr (WK > 1) __syncthreads();
    if (p.stamps) stamp[3] = __builtin_amdgcn_s_memrealtime();
    const int my_tiles = (ntl > k0) ? (ntl - k0 + kstep - 1) / kstep : 0;
    for (int j0 = 0; j0 < my_tiles; j0 += 64) {
      const int j = j0 + lane;
      bool take = false;
      if (j < my_tiles) {
        const int k = k0 + kstep * j;
        if (owner_of(k) != rank) {
          uint32_t* const cnt = cnt_of(tile_at(k));
          const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((old & kArrivals) == (uint32_t)(S - 1)) {
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            take = (old & kAbandon) != 0;
          }
        }
      }
      uint64_t m = __builtin_amdgcn_ballot_w64(take);
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        take_over(k0 + kstep * (j0 + b));
      }
    }
    if (tid == 0 && started_old == gridDim.x * gridDim.y - 1) {
      // Every workgroup of this launch has read the epoch: the next launch's.
      __hip_atomic_store(p.epoch + kCntStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.epoch, epoch0 + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    write_stamps();
    return;
  }

  if (p.pdefer) {
    // The partials held in LDS go out now, in one burst after the stream,
    // the workgroup's waves taking every WK-th tile (measured: mid-stream
    // partial stores slow the weight stream itself, T=32 K=7168 N=18432
    // 55-57 us without them against 63-65 us with). Tiles this rank owns
    // stay in LDS: their owner sums them from there.
    __syncthreads();  // every tile's partial is in LDS
    for (int k = wk; k < ntl; k += WK) {
      if (owner_of(k) == rank) continue;
      const int tile = tile_at(k);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, pbuf[(k * NT + tt) * 64 + lane]), pr,
                         p_off(rank, tile, tt));
    }
  }
  wait_vmem_all();  // this wave's partial stores are complete (coherent)
  if (p.stamps) stamp[3] = __builtin_amdgcn_s_memrealtime();
  int k0 = 0, kstep = 1;
  if constexpr (WK > 1) {
    __syncthreads();  // wave 0's stores, seen by every wave of the workgroup
    k0 = wk;
    kstep = WK;
  }
  // Sums the S partials of the tiles at list positions k0i (and k1i >= 0) in
  // rank order, one store each. With `held`, this rank's own partial is
  // taken from LDS (the owner's, which was never stored).
  auto finish = [&](int k0i, int k1i, bool held) {
    const int t0 = tile_at(k0i);
    const int t1c = k1i >= 0 ? tile_at(k1i) : t0;
    const int h0 = k0i;
    const int h1 = k1i >= 0 ? k1i : k0i;
#pragma unroll 1
    for (int tt = 0; tt < NT; ++tt) {
      const bool ok = in_t(tt);
      const bool ok1 = ok && k1i >= 0;
      f32x4 v0[8], v1[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < S) {
          const bool own = held && r == rank;
          v0[r] = __builtin_bit_cast(f32x4, ld16_coherent_if(ok && !own, pr, p_off(r, t0, tt)));
          v1[r] = __builtin_bit_cast(f32x4, ld16_coherent_if(ok1 && !own, pr, p_off(r, t1c, tt)));
          if (own) {
            v0[r] = pbuf[(h0 * NT + tt) * 64 + lane];
            v1[r] = pbuf[(h1 * NT + tt) * 64 + lane];
          }
        }
      }
      f32x4 s0 = v0[0], s1 = v1[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) {
        if (r < S) {
          s0 += v0[r];
          s1 += v1[r];
        }
      }
      store_quad(co, ok, s0, c_el(t0, tt));
      store_quad(co, ok1, s1, c_el(t1c, tt));
    }
  };
  // Finishes the tiles of the lanes set in `mask` (list position of lane b:
  // pos_of_lane(b)), two at a time.
  auto finish_mask = [&](uint64_t mask, auto pos_of_lane, bool held) {
    while (mask) {
      const int b0 = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int b1 = mask ? __builtin_ctzll(mask) : -1;
      if (b1 >= 0) mask &= mask - 1;
      finish(pos_of_lane(b0), b1 >= 0 ? pos_of_lane(b1) : -1, held);
    }
  };

  // Arrivals: this wave's share of the list, a lane per tile.
  const int my_tiles = (ntl > k0) ? (ntl - k0 + kstep - 1) / kstep : 0;
  for (int j0 = 0; j0 < my_tiles; j0 += 64) {
    const int j = j0 + lane;
    bool take = false;
    if (j < my_tiles) {
      const int k = k0 + kstep * j;
      const int tile = tile_at(k);
      const uint32_t old =
          __hip_atomic_fetch_add(cnt_of(tile), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // Last to arrive at a tile its owner gave up on: finish it here. That
      // includes a tile this workgroup owns: the arrival comes from wave
      // k mod WK, usually not the owner wave, and can land after the owner
      // wave has given up. Exactly one side finishes: the owner's fetch_or
      // saw all S arrivals, or the S-th arrival saw the abandon bit.
      take = (old & kAbandon) != 0 && (old & kArrivals) == (uint32_t)(S - 1);
      if (take) __hip_atomic_store(cnt_of(tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    handoff_order();  // the partial loads of a taken tile stay after the arrival
    finish_mask(__builtin_amdgcn_ballot_w64(take), [&](int b) { return k0 + kstep * (j0 + b); }, false);
  }

  if (p.stamps) stamp[5] = __builtin_amdgcn_s_memrealtime();
  // Owned tiles: k = k_first + S*m, m spread over the waves like the list.
  const int my_own = (n_own > k0) ? (n_own - k0 + kstep - 1) / kstep : 0;
  auto own_k = [&](int i) { return k_first + S * (k0 + kstep * i); };
  for (int i0 = 0; i0 < my_own; i0 += 64) {
    const int i = i0 + lane;
    const bool mine = i < my_own;
    const int tile = mine ? tile_at(own_k(i)) : 0;
    bool pending = mine;
    bool ready = false;
    const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.owner_wait;
    while (true) {
      if (pending) {
        const uint32_t v = __hip_atomic_load(cnt_of(tile), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & kArrivals) == (uint32_t)S) {
          ready = true;
          pending = false;
        }
      }
      if (__builtin_amdgcn_ballot_w64(pending) == 0) break;
      if (__builtin_amdgcn_s_memrealtime() > deadline) {
        if (p.pdefer) {
          // The tile may go to another rank now: its partial from this rank,
          // held in LDS so far, is stored (and complete) before the abandon.
          uint64_t pm = __builtin_amdgcn_ballot_w64(pending);
          while (pm) {
            const int b = __builtin_ctzll(pm);
            pm &= pm - 1;
            const int kk = own_k(i0 + b);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
              st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, pbuf[(kk * NT + tt) * 64 + lane]), pr,
                               p_off(rank, tile_at(kk), tt));
          }
          wait_vmem_all();
        }
        if (pending) {
          const uint32_t old = __hip_atomic_fetch_or(cnt_of(tile), kAbandon, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
          ready = (old & kArrivals) == (uint32_t)S;  // all arrived meanwhile: still ours
          pending = false;
          if (p.owner_wait > 0) note_timeout(p.health, (uint32_t)tile, (uint32_t)rank, p.owner_wait);
        }
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ready) __hip_atomic_store(cnt_of(tile), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.stamps) stamp[6] = __builtin_amdgcn_s_memrealtime();
    handoff_order();  // the partial loads stay after the poll that saw every arrival
    finish_mask(__builtin_amdgcn_ballot_w64(ready), [&](int b) { return own_k(i0 + b); }, p.pdefer != 0);
  }
  write_stamps();
}

// ---------------------------------------------------------------------------
// configurations and dispatch
// ---------------------------------------------------------------------------

namespace {

struct Shape {
  int rg, wk, wn, d, c;
  int max_nt;     // largest token-tile count this shape is built for (bf16)
  int max_nt_mx;  // the same for block-scaled weights (their decode needs registers)
};

// The instantiated workgroup shapes (each for NT = 1..8 and both weight
// formats; MXFP4 ignores c: one 16-byte load is a whole scale block).
constexpr Shape kShapes[] = {
    {1, 4, 1, 8, 2, 4, 4},  // 0: 16 rows, 4 waves along K, 2 pieces per lane per step
    {1, 8, 1, 8, 2, 4, 4},  // 1: 16 rows, 8 waves along K
    {1, 8, 1, 8, 1, 4, 4},  // 2: 16 rows, 8 waves along K, 1 piece per step
    {2, 2, 2, 4, 1, 8, 8},  // 3: 64 rows, two wave columns share the staged X (large T)
    {1, 4, 2, 8, 2, 4, 4},  // 4: 32 rows, two wave columns share the staged X
    {1, 2, 1, 4, 1, 8, 8},  // 5: 16 rows, any T: the fallback when no larger tile divides N
    {2, 1, 8, 4, 1, 8, 6},  // 6: 256 rows, eight wave columns share the staged X (large T)
    {2, 1, 4, 4, 1, 8, 6},  // 7: 128 rows, four wave columns share the staged X
};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

constexpr int kMaxXLds = 128 * 1024;  // LDS for the staged X slice (or chunk)
constexpr int kMaxLds = 159 * 1024;   // dynamic LDS per workgroup (160 KiB per CU on gfx950)

template <int NT, int SH, int WF>
hipError_t launch_one(const Tactic& t, const GemmParams& p, hipStream_t s) {
  constexpr Shape sh = kShapes[SH];
  if constexpr (NT > (WF != kBf16 ? sh.max_nt_mx : sh.max_nt)) {
    return hipErrorInvalidValue;  // not built: pick_tactic never selects it
  } else {
    auto kern = splitk_gemm_kernel<NT, sh.rg, sh.wk, sh.wn, sh.d, sh.c, WF>;
    hipLaunchKernelGGL(kern, dim3(t.grid, p.L), dim3(t.threads), t.lds, s, p);
    return hipGetLastError();
  }
}

template <int NT, int WF>
hipError_t launch_nt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (sh) {
    case 0: return launch_one<NT, 0, WF>(t, p, s);
    case 1: return launch_one<NT, 1, WF>(t, p, s);
    case 2: return launch_one<NT, 2, WF>(t, p, s);
    case 3: return launch_one<NT, 3, WF>(t, p, s);
    case 4: return launch_one<NT, 4, WF>(t, p, s);
    case 5: return launch_one<NT, 5, WF>(t, p, s);
    case 6: return launch_one<NT, 6, WF>(t, p, s);
    case 7: return launch_one<NT, 7, WF>(t, p, s);
  }
  return hipErrorInvalidValue;
}

template <int WF>
hipError_t launch_fmt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.nt) {
    case 1: return launch_nt<1, WF>(sh, t, p, s);
    case 2: return launch_nt<2, WF>(sh, t, p, s);
    case 3: return launch_nt<3, WF>(sh, t, p, s);
    case 4: return launch_nt<4, WF>(sh, t, p, s);
    case 5: return launch_nt<5, WF>(sh, t, p, s);
    case 6: return launch_nt<6, WF>(sh, t, p, s);
    case 7: return launch_nt<7, WF>(sh, t, p, s);
    case 8: return launch_nt<8, WF>(sh, t, p, s);
  }
  return hipErrorInvalidValue;
}

int shape_index(const Tactic& t) {
  for (int i = 0; i < kNumShapes; ++i)
    if (kShapes[i].rg == t.rg && kShapes[i].wk == t.wk && kShapes[i].wn == t.wn &&
        kShapes[i].d == t.d && kShapes[i].c == t.c)
      return i;
  return -1;
}

// Largest chunk kc that divides ks, is a multiple of `step` and whose staged
// X tile (T rows of bf16) fits in the LDS budget. ks == 0 gives 0 (no chunk).
int pick_kc(int ks, int step, int T) {
  if (ks == 0) return 0;
  if (ks % step) return -1;
  const int units = ks / step;
  for (int m = 1; m <= units; ++m) {
    if (units % m) continue;
    const int kc = ks / m;
    if ((long)T * kc * 2 <= kMaxXLds) return kc;
  }
  return -1;
}

// Fills the launch geometry of shape `si`; false if it does not fit.
bool shape_fits(int si, int T, int N, int ks, int S, int wf, Tactic* t) {
  const bool mx = wf != kBf16;
  const Shape& c = kShapes[si];
  if (t->nt > (mx ? c.max_nt_mx : c.max_nt)) return false;
  const int tile_n = 16 * c.rg * c.wn;
  if (N % tile_n) return false;
  const int step = mx ? 4 * lane_k(wf) : 32 * c.c;
  const int kc = pick_kc(ks, step, T);
  if (kc < 0) return false;
  const int x_lds = T * kc * 2;
  const int red_lds = (c.wk - 1) * c.wn * c.rg * t->nt * 64 * 16;
  const int lds = x_lds > red_lds ? x_lds : red_lds;
  if (lds > kMaxLds) return false;
  t->rg = c.rg;
  t->wk = c.wk;
  t->wn = c.wn;
  t->d = c.d;
  t->c = c.c;
  t->tile_n = tile_n;
  t->threads = 64 * c.wk * c.wn;
  t->kc = kc;
  t->lds = lds;
  t->grid = (N / tile_n) * S;
  t->kind = 0;
  t->shape = si;
  return true;
}

}  // namespace

// ---- persistent stream kernel configurations --------------------------

struct StreamShape {
  int wk, wn, d, c, mode;
};
constexpr StreamShape kStreamShapes[] = {
    {8, 1, 8, 2, kStreamDeferred},  // 0: 8 waves share each tile's K slice, deferred hand-off
    {8, 1, 8, 1, kStreamDeferred},  // 1
    {8, 1, 8, 2, kStreamEpilogue},  // 2: 7 streaming waves + an epilogue wave (pipelined hand-off)
    {8, 1, 8, 1, kStreamEpilogue},  // 3
    {4, 1, 8, 1, kStreamDeferred},  // 4
    {1, 8, 8, 2, kStreamDeferred},  // 5: 8 waves, each streaming its own tiles
    {8, 1, 8, 2, kStreamStorer},    // 6: 7 streaming waves + a storer wave
};
constexpr int kNumStreamShapes = sizeof(kStreamShapes) / sizeof(kStreamShapes[0]);

// Load steps in flight per streaming wave. The storer shape on bf16 weights
// (one line pair per step) keeps fewer than the table's 8: with seven waves
// streaming one tile's rows, a shallower ring reads the same bytes faster
// (bit-identical; one box, two runs each, cold single launches: K=N=16384
// T=1/8/16 86.4-87.7 -> 85.8-86.8 us with 3 steps, T=32 92.2-92.3 ->
// 90.7 us and T=32 K=7168 N=18432 55.0-55.2 -> 54.3-54.9 us with 4; 2 steps
// lose 3-4 us at two token tiles, 10 steps lose about 1 us everywhere).
constexpr int stream_depth(const StreamShape& sh, int nt, int wf) {
  return (sh.mode == kStreamStorer && wf == kBf16 && sh.c == 2) ? (nt == 1 ? 3 : 4) : sh.d;
}
constexpr int kStreamMaxNT = 2;
constexpr int kStreamMaxX = 128 * 1024;
constexpr int kClusterMaxGrid = 512;
constexpr long kClusterMaxBatchGrid = 8192;

template <int NT, int SH, int WF>
hipError_t launch_stream_one(const Tactic& t, const GemmParams& p, hipStream_t s) {
  constexpr StreamShape sh = kStreamShapes[SH];
  auto kern = splitk_stream_kernel<NT, sh.wk, sh.wn, stream_depth(sh, NT, WF), sh.c, sh.mode, WF>;
  hipLaunchKernelGGL(kern, dim3(t.grid, p.L), dim3(t.threads), t.lds, s, p);
  return hipGetLastError();
}

template <int NT, int WF>
hipError_t launch_stream_nt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (sh) {
    case 0: return launch_stream_one<NT, 0, WF>(t, p, s);
    case 1: return launch_stream_one<NT, 1, WF>(t, p, s);
    case 2: return launch_stream_one<NT, 2, WF>(t, p, s);
    case 3: return launch_stream_one<NT, 3, WF>(t, p, s);
    case 4: return launch_stream_one<NT, 4, WF>(t, p, s);
    case 5: return launch_stream_one<NT, 5, WF>(t, p, s);
    case 6: return launch_stream_one<NT, 6, WF>(t, p, s);
  }
  return hipErrorInvalidValue;
}

template <int WF>
hipError_t launch_stream_fmt(int sh, const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.nt) {
    case 1: return launch_stream_nt<1, WF>(sh, t, p, s);
    case 2: return launch_stream_nt<2, WF>(sh, t, p, s);
  }
  return hipErrorInvalidValue;
}

// Fills the geometry of persistent shape `si`; false if it does not apply.
bool stream_fits(int si, int T, int N, int ks, int S, int wf, Tactic* t, int L = 1) {
  const StreamShape& c = kStreamShapes[si];
  if (t->nt > kStreamMaxNT || ks == 0) return false;
  // This kernel addresses all N weight rows (and their scales) through one
  // buffer resource with 32-bit offsets: the span must stay below 2^31 bytes,
  // where the out-of-range offset kOOB lies beyond every valid one. Larger
  // weight matrices go to the kernels that rebase per tile.
  const uint64_t K = (uint64_t)ks * (uint64_t)S;
  if ((uint64_t)N * row_bytes(wf, (uint32_t)K) >= kOOB) return false;
  if (wf != kBf16 && (uint64_t)N * (K / 32) >= kOOB) return false;
  // K elements per ring slot: one step of two pieces, or two one-piece steps.
  const int step = wf != kBf16 ? 2 * 4 * lane_k(wf) : 64;
  if (ks % step) return false;
  const int cs = ks / step;
  const int streaming = c.mode == kStreamDeferred ? c.wk : c.wk - 1;
  if (cs < streaming) return false;  // every streaming wave needs a slot per tile
  // The storer organisation is built for one workgroup per CU (single problems).
  if (c.mode == kStreamStorer && L != 1) return false;
  const long x_lds = (long)T * ks * 2;
  if (x_lds > kStreamMaxX) return false;
  const int parked = c.wk - 1;  // sums parked in LDS per tile
  const int red = c.wk > 1 ? 2 * parked * t->nt * 64 * 16 : 0;
  const long lds = x_lds + red;
  if (lds > kMaxLds) return false;
  const int n_tiles = N / 16;
  // Resident workgroups per CU: LDS-bound and the register budget the kernel
  // is built with.
  const int waves = c.wk * c.wn;
  int per_cu = (int)((160L * 1024) / (lds > 0 ? lds : 1));
  if (per_cu > stream_wgs_per_cu(t->nt)) per_cu = stream_wgs_per_cu(t->nt);
  // A single problem runs best with one workgroup per CU (measured: as fast
  // or faster on every decode and sweep shape, up to 40 % at T=24..32,
  // N=2048); batches keep the residency the LDS allows.
  if (L == 1) per_cu = 1;
  per_cu = knob(kKnobWgPerCu, per_cu);
  if (per_cu < 1) per_cu = 1;
  long g = ((long)kChipCUs * per_cu) / ((long)S * (L > 0 ? L : 1));  // the whole batch resident
  const long g_max = (n_tiles + c.wn - 1) / c.wn;  // every column gets a tile
  if (g > g_max) g = g_max;
  if (g < 1) g = 1;
  t->kind = 1;
  t->rg = 1;
  t->wk = c.wk;
  t->wn = c.wn;
  t->d = stream_depth(c, t->nt, wf);
  t->c = c.c;
  t->tile_n = 16;
  t->threads = 64 * waves;
  t->kc = ks;
  t->lds = (int)lds;
  t->grid = (int)g * S;
  t->shape = si;
  t->resident = per_cu;
  // Partials held in LDS until the stream ends, where they fit beside the
  // activation slice (single problems, waves sharing each tile, split K).
  t->pdefer = 0;
  if (L == 1 && S > 1 && c.wk > 1 && c.wn == 1 && c.mode != kStreamEpilogue &&
      knob(kKnobPdefer, 1) != 0) {
    const long per_wg = (n_tiles + g - 1) / g;  // tiles of the busiest workgroup
    const long pl = per_wg * t->nt * 64 * 16;
    if (lds + pl <= kMaxLds) {
      t->pdefer = 1;
      t->lds = (int)(lds + pl);
    }
  }
  return true;
}

bool pick_tactic(int T, int N, int K, int S, int wf, Tactic* out, int L) {
  const bool mx = wf != kBf16;
  Tactic t{};
  t.nt = (T + 15) / 16;
  if (t.nt < 1) t.nt = 1;
  if (t.nt > 8) return false;
  t.wf = wf;
  const int ks = K / S;
  const int tr = T > 0 ? T : 1;

  // A pinned kind (kKnobKind: tests and tuning runs) restricts the choice to
  // that kernel kind; kKnobFold and kKnobClusterC cap the fold and pin the
  // pieces per lane of kind 2.
  const int kind = knob(kKnobKind, -1);
  if (kind == 2 || kind < 0) {
    Tactic c = t;
    if (cluster_fits(tr, N, ks, S, wf, knob(kKnobFold, 8), knob(kKnobClusterC, 0), &c, L)) {
      // Whole tiles per workgroup pay off while the grid is about one
      // workgroup per CU; beyond, the persistent kernel's staged activations
      // and amortised ramp-up win. Every cluster workgroup re-reads all of X
      // from L2, T*2 bytes per tile row against the row's weight bytes; in a
      // batch the cluster kernel stays only while that is small (measured:
      // T=1 K=1024 N=1024 batches run 1.1 vs 1.6 us a problem on it, the
      // T=8 K=7168 N=2048 ones 9.6 vs 6.4 us on the persistent kernel).
      // An unfolded tile with fewer workgroups than CUs leaves the chip
      // partly idle; the persistent kernel then wins (measured T=12..32,
      // N=1024..2048: 9.6-15.6 us against 12.1-18.3 us). Folded tiles stay
      // ahead even there (T=5..8, N=1024).
      const double x_per_w = (double)tr * 2.0 / ((double)c.tile_n * weight_bytes_per_elem(wf));
      const bool fills = c.fold >= 2 || c.grid >= kChipCUs;
      const bool small = L == 1 ? (c.grid <= kClusterMaxGrid && fills)
                                : (x_per_w <= 0.5 && (long)c.grid * L <= kClusterMaxBatchGrid);
      if (kind == 2 || small) {
        *out = c;
        return true;
      }
    }
    if (kind == 2) return false;
  }
  // Persistent streaming kernel (a pinned kKnobStream forces one of its
  // shapes, for tests and tuning runs).
  if (kind == 1 || kind < 0) {
    const int forced = knob(kKnobStream, -1);
    if (forced >= 0) {
      if (forced < kNumStreamShapes && stream_fits(forced, tr, N, ks, S, wf, &t, L)) {
        *out = t;
        return true;
      }
    } else {
      // Eight waves share each tile's K slice (measured fastest on the decode
      // shapes: 16 weight rows open per workgroup, 8 streams on them); the
      // one-wave-per-tile shapes remain for when the slice is too short.
      // With few tiles per workgroup the hand-off is most of the tail, and a
      // dedicated epilogue wave that overlaps it with the stream wins; with
      // many tiles all eight waves streaming wins.
      // Single problems with many tiles per workgroup: 7 streaming waves and
      // a storer wave, which takes each tile's wave-order sum and its partial
      // off the streaming waves (measured with partials held in LDS:
      // K=N=16384 T=1 / 8 / 16 85.0-85.6 / 87.2-88.3 / 89.9-90.3 us against
      // 87.3-87.8 / 89.4-89.7 / 91.3 us with 8 streaming waves; T=32
      // K=7168 N=18432 57.3 against 62.2-62.5 us). Where the storer shape
      // does not fit (batches, slices of fewer than 7 ring slots per tile),
      // 8 streaming waves.
      static const int many[] = {6, 0, 1, 2, 3, 4, 5};
      static const int few[] = {2, 3, 0, 1, 4, 5, 6};
      const int* pref = many;
      bool held = true;  // the preferred shape holds its partials in LDS (or needs none)
      for (int mi = 0; mi < kNumStreamShapes; ++mi) {
        const int si = many[mi];
        Tactic probe = t;
        if (stream_fits(si, tr, N, ks, S, wf, &probe, L)) {
          const int groups = probe.grid / S;
          const int per_wg = (N / 16 + groups - 1) / groups;
          if (per_wg <= 4) pref = few;
          held = S == 1 || probe.pdefer != 0;
          break;
        }
      }
      // Where the partials do not fit in LDS, the storer wave holds them in
      // its registers and stores them in bursts (K=N=16384 T=24/32).
      if (pref == many && !held && stream_fits(6, tr, N, ks, S, wf, &t, L)) {
        *out = t;
        return true;
      }
      for (int oi = 0; oi < kNumStreamShapes; ++oi) {
        const int si = pref[oi];
        if (stream_fits(si, tr, N, ks, S, wf, &t, L)) {
          *out = t;
          return true;
        }
      }
    }
  }
  if (kind == 1) return false;
  // Many tokens: the wide-tile kernel with double-buffered X chunks.
  if (kind == 3 || kind < 0) {
    if (wide_fits(tr, N, ks, S, wf, &t)) {
      *out = t;
      return true;
    }
    if (kind == 3) return false;
  }
  // A tiled shape pinned for tests and tuning runs (kKnobShape), if it fits.
  if (const int si = knob(kKnobShape, -1); si >= 0) {
    if (si < kNumShapes && shape_fits(si, tr, N, ks, S, wf, &t)) {
      *out = t;
      return true;
    }
  }
  // Preference order: up to 32 tokens, 16-row tiles with 8 waves on each
  // (few DRAM pages open per workgroup, deep prefetch); beyond, the widest
  // tile whose wave columns share the staged activations (each workgroup
  // reads its K range of X from L2, so wider tiles mean less of that traffic).
  static const int small_t[] = {1, 2, 0, 4, 3, 5, 7, 6};
  static const int large_t[] = {6, 7, 3, 4, 1, 2, 0, 5};
  static_assert(sizeof(small_t) / sizeof(int) == kNumShapes && sizeof(large_t) / sizeof(int) == kNumShapes,
                "every shape appears in both orders");
  const int* order = (t.nt <= 2) ? small_t : large_t;
  for (int oi = 0; oi < kNumShapes; ++oi) {
    if (shape_fits(order[oi], tr, N, ks, S, wf, &t)) {
      *out = t;
      return true;
    }
  }
  return false;
}

bool tactic_mailbox(const Tactic& t) {
  return t.kind == 1 && kStreamShapes[t.shape].mode != kStreamEpilogue;
}

hipError_t launch_gemm(const Tactic& t, const GemmParams& p, hipStream_t s) {
  if (t.kind == 3) return launch_wide(t, p, s);
  if (t.kind == 2) return launch_cluster(t, p, s);
  if (t.kind == 1) {
    switch (t.wf) {
      case kBf16: return launch_stream_fmt<kBf16>(t.shape, t, p, s);
      case kMxfp4: return launch_stream_fmt<kMxfp4>(t.shape, t, p, s);
      case kMxfp8: return launch_stream_fmt<kMxfp8>(t.shape, t, p, s);
    }
    return hipErrorInvalidValue;
  }
  const int sh = shape_index(t);
  if (sh < 0) return hipErrorInvalidValue;
  switch (t.wf) {
    case kBf16: return launch_fmt<kBf16>(sh, t, p, s);
    case kMxfp4: return launch_fmt<kMxfp4>(sh, t, p, s);
    case kMxfp8: return launch_fmt<kMxfp8>(sh, t, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skg
