// Split-K GEMM kernel for many tokens (T = 33..128): wide weight tiles,
// activations staged in double-buffered K chunks.
//
// Same method as the other kernels (page
// vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk, module
// summary and SplitKGemm): rank r accumulates the contiguous K slice r in
// FP32, the ranks' partials are summed once in rank order, rounded to bf16
// (RNE) and stored once.
//
// With up to 128 tokens the activation slice no longer fits in LDS, and
// every workgroup that multiplies a weight tile must read the activations of
// its K range from L2. That traffic is (N / rows per workgroup) * T * K * 2
// bytes, so the tile is wide: 256 weight rows, eight waves of 32 rows each
// (two MFMA row groups), all sharing one staged activation chunk.
//  * X moves through LDS in chunks of KC elements, double-buffered: the loads
//    of chunk c + 1 go out at the start of chunk c, into registers, and are
//    written to the other buffer when chunk c is done; one barrier per chunk.
//  * Each wave streams its 32 weight rows over the whole K slice through a
//    register ring that runs on across chunk boundaries (weights do not
//    depend on the chunk). A slot holds two load steps as whole-line loads
//    (rows 0-7 and 8-15 of each 16-row group over both steps' 64-byte
//    windows), rearranged into MFMA A operands at use.
//  * Hand-off per wave column (32 rows x T): the column's partial goes to
//    the workspace with device-coherent stores, the wave bumps the column's
//    arrival counter, and one owner rank per column, (column + tile) mod S,
//    waits for the other ranks (bounded), sums the partials in rank order and
//    stores C. An owner that runs out of time sets an abandon bit and the
//    last rank to arrive finishes the column instead.

#include "device/mfma.h"
#include "device/out.h"
#include "device/pack.h"
#include "device/types.h"
#include "device/wfmt.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

constexpr int kWideWaves = 8;                // wave columns per workgroup
constexpr int kWideRows = 32 * kWideWaves;   // weight rows per workgroup
// bf16 tiles of up to 64 tokens keep three activation chunks in LDS with a
// handshake (below); the others two, closed by a barrier.
constexpr bool wide_drift(int nt, int wf) { return wf == kBf16 && nt <= 4; }
constexpr int wide_kc(int nt, int wf) {  // K elements per X chunk
  return wide_drift(nt, wf) ? 256 : (nt <= 4 ? 512 : 256);
}
constexpr int wide_nbuf(int nt, int wf) { return wide_drift(nt, wf) ? 3 : 2; }

}  // namespace

template <int NT, int WF>
__global__ __launch_bounds__(64 * kWideWaves) void splitk_wide_kernel(GemmParams p) {
  select_problem(p);
  constexpr bool MX = WF != kBf16;            // block-scaled weights
  constexpr int LK = lane_k(WF);              // K elements of one lane's 16-byte piece
  constexpr int RG = 2;                       // 16-row groups per wave
  constexpr int THREADS = 64 * kWideWaves;
  constexpr int SUBS = MX ? LK / 8 : 1;       // MFMA K-steps per load step
  constexpr int STEP_K = MX ? 4 * LK : 32;    // K elements of one load step
  constexpr int KC = wide_kc(NT, WF);
  constexpr bool DRIFT = wide_drift(NT, WF);
  constexpr int NB = wide_nbuf(NT, WF);  // activation chunk buffers in LDS
  constexpr int CS = KC / STEP_K;             // load steps per chunk
  // A ring slot holds two load steps: per 16-row group, rows 0-7 and rows
  // 8-15 over both steps' 64-byte windows, one whole 128-byte line per row
  // and instruction (non-temporal), rearranged into the two steps' operands
  // at use.
  constexpr int CS2 = CS / 2;                 // ring slots per chunk
  static_assert(CS % 2 == 0, "a chunk holds whole step pairs");
  // Ring depth in slots (divides CS2): 2 slots = 8 KiB of weights in flight
  // per wave. With 256 rows streaming per workgroup, more requests in flight
  // do not read the same bytes any faster (bf16, bit-identical, cold single
  // launches, one box, three runs each against 4 slots: K=N=16384 T=64
  // 117.8 against 118.0 us, T=128 126.4 against 127.6 us; 1 slot is slower,
  // 125-133 us).
  constexpr int D = CS2 < 2 ? CS2 : 2;
  static_assert(CS2 % D == 0, "ring slots repeat every chunk");

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  uint64_t stamp[5];  // optional phase stamps (s_memrealtime, 100 MHz)
  stamp[0] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = tid >> 6;
  const int g = lane >> 4;
  const int li = lane & 15;

  const int S = p.S;
  const int T = p.T;
  const int K = p.K;
  const int N = p.N;
  const int tile = blockIdx.x / S;
  const int rank = blockIdx.x - tile * S;
  const int n0 = tile * kWideRows;
  const int kbase = rank * p.ks;
  const int nchunks = p.ks / KC;
  const int total = nchunks * CS2;  // ring slots (step pairs) of this wave

  const uint32_t wrow_bytes = row_bytes(WF, (uint32_t)K);
  const rsrc_t wr = make_rsrc(static_cast<const uint8_t*>(p.w) + (size_t)n0 * wrow_bytes,
                              (uint32_t)kWideRows * wrow_bytes);
  const rsrc_t sr = MX ? make_rsrc(p.wscale + (size_t)n0 * (K / 32), (uint32_t)kWideRows * (uint32_t)(K / 32))
                       : wr;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)T * (uint32_t)K * 2u);

  uint32_t row_off[RG], srow_off[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const uint32_t row0 = (uint32_t)((wn * RG + rg) * 16);
    row_off[rg] = row0 * wrow_bytes + line_pair_offset(li, 0, wrow_bytes);
    srow_off[rg] = (row0 + (uint32_t)li) * (uint32_t)(K / 32);  // scales: operand layout
  }

  // ---- weight ring ----------------------------------------------------------
  u32x4 ring[D][RG][2];
  uint32_t sring[D][RG][2];
  auto issue = [&](int slot, int q) {
    const bool ok = q < total;
    const int kel = kbase + q * 2 * STEP_K;
    const uint32_t lo = elem_byte(WF, (uint32_t)kel) + 16u * g;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
      for (int h = 0; h < 2; ++h) ring[slot][rg][h] = ld16_if<kPolicyStream>(ok, wr, row_off[rg] + lo + 8u * wrow_bytes * h);
      if constexpr (MX) {
#pragma unroll
        for (int w = 0; w < 2; ++w)
          sring[slot][rg][w] = ld1_if(ok, sr, srow_off[rg] + (uint32_t)((kel + w * STEP_K + LK * g) / 32));
      }
    }
  };

  // ---- X chunks -------------------------------------------------------------
  // Loads take 16-byte pieces K fastest (piece pc: token pc / (KC / 8),
  // K offset 8 * (pc % (KC / 8))), so every 4-lane group reads one
  // contiguous run. Operand-ordered layout of one chunk over TP = 16 * NT
  // token slots: slot
  // ((j*SUBS + s)*4 + gg)*TP + t holds token t's 8 elements of load step j,
  // sub-step s, lane K block gg. Slots of tokens t >= T hold zeros (their
  // loads are out of range and read zero without a memory access), and every
  // LDS offset is a compile-time constant.
  constexpr int TP = 16 * NT;
  constexpr int CHUNK_BYTES = TP * KC * 2;
  constexpr int PIECES = TP * (KC / 8);
  constexpr int XP = (PIECES + THREADS - 1) / THREADS;  // pieces per thread per chunk
  auto x_slot = [&](int j, int s, int gg, int t) -> int { return ((j * SUBS + s) * 4 + gg) * TP + t; };
  u32x4 xreg[XP];
  auto x_load = [&](int c, u32x4 (&dst)[XP]) {
    const int k0 = kbase + c * KC;
#pragma unroll
    for (int b = 0; b < XP; ++b) {
      const int pc = tid + b * THREADS;
      const int t = pc / (KC / 8);
      const int k = (pc % (KC / 8)) * 8;
      dst[b] = ld16_if(pc < PIECES && t < T, xr, ((uint32_t)t * (uint32_t)K + (uint32_t)(k0 + k)) * 2u);
    }
  };
  auto x_store = [&](int c, const u32x4 (&src)[XP]) {
    uint8_t* buf = smem + (c % NB) * CHUNK_BYTES;
#pragma unroll
    for (int b = 0; b < XP; ++b) {
      const int pc = tid + b * THREADS;
      if (PIECES % THREADS == 0 || pc < PIECES) {
        const int t = pc / (KC / 8);
        const int k = (pc % (KC / 8)) * 8;
        int j, s2, gg;
        if constexpr (MX) {
          j = k / STEP_K; gg = (k % STEP_K) / LK; s2 = (k % LK) / 8;
        } else {
          j = k / 32; s2 = 0; gg = (k % 32) / 8;
        }
        *reinterpret_cast<u32x4*>(buf + x_slot(j, s2, gg, t) * 16) = src[b];
      }
    }
  };

  f32x4 acc[RG][NT];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slot jp of chunk c: load steps 2*jp and 2*jp + 1 of the chunk.
  auto compute = [&](int slot, int c, int jp) {
    const uint8_t* buf = smem + (c % NB) * CHUNK_BYTES;
    u32x4 a[RG][2];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) line_pair_to_operands(ring[slot][rg][0], ring[slot][rg][1], a[rg][0], a[rg][1]);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int j = 2 * jp + w;
#pragma unroll
      for (int s2 = 0; s2 < SUBS; ++s2) {
        bf16x8 b[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          b[tt] = as_bf16x8(*reinterpret_cast<const u32x4*>(buf + x_slot(j, s2, g, tt * 16 + li) * 16));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          bf16x8 af;
          if constexpr (MX) {
            af = decode_operand<WF>(a[rg][w], s2, e8m0_f32(sring[slot][rg][w]));
          } else {
            af = as_bf16x8(a[rg][w]);
          }
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[rg][tt] = mfma_bf16(af, b[tt], acc[rg][tt]);
        }
      }
    }
  };

  if constexpr (!DRIFT) {
    // Prologue: chunk 0's X first (its LDS writes then wait only for X), the
    // weight ring behind it.
    x_load(0, xreg);
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s, s);
    x_store(0, xreg);
    __syncthreads();
    stamp[1] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

    for (int c = 0; c < nchunks; ++c) {
      const bool next = c + 1 < nchunks;
      if (next) x_load(c + 1, xreg);
#pragma unroll
      for (int jp = 0; jp < CS2; ++jp) {
        const int slot = jp % D;
        compute(slot, c, jp);
        issue(slot, c * CS2 + jp + D);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (next) {
        x_store(c + 1, xreg);
        __syncthreads();
      }
    }
  } else {
    // Three chunk buffers and a handshake instead of a barrier per chunk:
    // chunk c sits in buffer c % 3, a wave computes it once all eight waves
    // have stored their part of it (ready), and a wave stores chunk c + 2 at
    // the end of chunk c once all eight have finished chunk c - 1, the
    // buffer's previous user (done). A wave can so run up to a chunk ahead
    // of the slowest one; with one barrier per chunk every chunk waited for
    // the slowest wave (measured: a timing copy without those barriers ran
    // 117.5 against 127.4 us at T=64, K=N=16384). Both counts only grow: the
    // u-th use of a buffer (u = c / 3) is ready at 8 (u + 1) stores and free
    // again at 8 (u + 1) finished computes. A wait that runs out (not
    // expected: the waves of a workgroup run together) is recorded in the
    // health words and the wave goes on.
    __shared__ uint32_t chunk_ready[3], chunk_done[3];
    auto signal = [&](uint32_t* ctr) {
      if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto wait_at_least = [&](uint32_t* ctr, uint32_t target, uint32_t what) {
      const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + 1000000;  // 10 ms
      while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (__builtin_amdgcn_s_memrealtime() > deadline) {
          if (lane == 0) note_timeout(p.health, 0xFFFFFFFEu, what, 1000000u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    // Prologue: chunks 0 and 1, their X loads ahead of the weight ring (so
    // their LDS writes wait only for X), made visible by one barrier.
    u32x4 xreg1[XP];
    x_load(0, xreg);
    if (nchunks > 1) x_load(1, xreg1);
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s, s);
    x_store(0, xreg);
    if (nchunks > 1) x_store(1, xreg1);
    if (tid < 3) {
      chunk_ready[tid] = tid < 2 ? 8u : 0u;  // chunks 0 and 1 are stored before the barrier
      chunk_done[tid] = 0u;
    }
    __syncthreads();
    stamp[1] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

    for (int c = 0; c < nchunks; ++c) {
      const bool ahead = c + 2 < nchunks;
      if (ahead) x_load(c + 2, xreg);
      if (c >= 2) wait_at_least(&chunk_ready[c % 3], 8u * (uint32_t)(c / 3 + 1), (uint32_t)c);
#pragma unroll
      for (int jp = 0; jp < CS2; ++jp) {
        const int slot = jp % D;
        compute(slot, c, jp);
        issue(slot, c * CS2 + jp + D);
        __builtin_amdgcn_sched_barrier(0);
      }
      signal(&chunk_done[c % 3]);  // this wave's reads of chunk c are complete
      if (ahead) {
        // Buffer (c + 2) % 3 last held chunk c - 1.
        if (c >= 1) wait_at_least(&chunk_done[(c + 2) % 3], 8u * (uint32_t)((c - 1) / 3 + 1), (uint32_t)c);
        x_store(c + 2, xreg);
        signal(&chunk_ready[(c + 2) % 3]);
      }
    }
  }

  stamp[2] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  // Thread 0 (wave 0) writes the stamps: entry, first chunk staged, weight
  // stream done, its column's partial stored, exit.
  auto write_stamps = [&]() {
    if (p.stamps != nullptr && tid == 0) {
      stamp[4] = __builtin_amdgcn_s_memrealtime();
      const rsrc_t sr8 = make_rsrc(p.stamps + (size_t)blockIdx.x * 8, 64);
#pragma unroll
      for (int i = 0; i < 5; ++i)
        st8_if(true, u32x2{(uint32_t)stamp[i], (uint32_t)(stamp[i] >> 32)}, sr8, 8u * i);
    }
  };

  // ---- output ------------------------------------------------------------------
  const int n_lane = n0 + wn * RG * 16 + 4 * g;  // feature of quad element 0, rg = 0
  const COut co = make_cout(p);
  auto c_el = [&](int rg, int tt) -> uint32_t {
    return (uint32_t)(tt * 16 + li) * (uint32_t)N + (uint32_t)(n_lane + rg * 16);
  };
  auto in_t = [&](int tt) -> bool { return tt * 16 + li < T; };
  if (S == 1) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) store_quad(co, in_t(tt), acc[rg][tt], c_el(rg, tt));
    stamp[3] = stamp[2];
    write_stamps();
    return;
  }

  // ---- hand-off of this wave's column ------------------------------------------
  // Partials: FP32, tile-major [S, N/16, T, 16] (rank r's partial of one
  // 16-row group is T x 64 contiguous bytes), so a wave's store or read-back
  // of a token tile covers whole lines.
  const rsrc_t pr = make_rsrc(p.part, (uint32_t)S * (uint32_t)T * (uint32_t)N * 4u);
  const uint32_t grp0 = (uint32_t)(n0 / 16 + wn * RG);  // this wave's first 16-row group
  auto p_off = [&](int r, int rg, int tt) -> uint32_t {
    return (((uint32_t)r * (uint32_t)(N / 16) + grp0 + (uint32_t)rg) * (uint32_t)T + (uint32_t)(tt * 16 + li)) * 64u +
           16u * (uint32_t)g;
  };
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      st16_coherent_if(in_t(tt), __builtin_bit_cast(u32x4, acc[rg][tt]), pr, p_off(rank, rg, tt));
  wait_vmem_all();  // the column's partial is complete (coherent) before it is announced
  stamp[3] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

  constexpr uint32_t kArrivals = 0xFFu;
  constexpr uint32_t kAbandon = 0x100u;
  uint32_t* cnt = p.cnt + (size_t)(n0 / 16 + wn * RG) * kCntStride;  // one 128-byte line each
  const bool owner = (wn + tile) % S == rank;
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  bool finish = false;
  if (owner) {
    if ((old & kArrivals) == (uint32_t)(S - 1)) {
      finish = true;  // the others were all here already
    } else {
      const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.owner_wait;
      while (true) {
        uint32_t v = 0;
        if (lane == 0) v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = __builtin_amdgcn_readfirstlane(v);
        if ((v & kArrivals) == (uint32_t)S) {
          finish = true;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() > deadline) {
          uint32_t o2 = 0;
          if (lane == 0) {
            o2 = __hip_atomic_fetch_or(cnt, kAbandon, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (p.owner_wait > 0)
              note_timeout(p.health, (uint32_t)(n0 / 16 + wn * RG), (uint32_t)rank, p.owner_wait);
          }
          o2 = __builtin_amdgcn_readfirstlane(o2);
          finish = (o2 & kArrivals) == (uint32_t)S;  // all arrived meanwhile: still ours
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  } else {
    // Last to arrive at a column its owner gave up on: finish it here.
    finish = (old & kAbandon) != 0 && (old & kArrivals) == (uint32_t)(S - 1);
  }
  if (!finish) {
    write_stamps();
    return;
  }
  if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  handoff_order();  // the partial loads below stay after the arrivals were seen

  // Rank-order sum (this rank's partial from registers), one bf16 store per
  // quad. BATCH quads at a time keep BATCH * (S - 1) loads in flight.
  constexpr int PAIRS = RG * NT;
  auto reduce = [&]<int BATCH, int OTHERS>() {
#pragma unroll
    for (int p0 = 0; p0 < PAIRS; p0 += BATCH) {
      f32x4 v[BATCH][OTHERS];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        if (p0 + b < PAIRS) {
          const int rg = (p0 + b) / NT, tt = (p0 + b) % NT;
#pragma unroll
          for (int r = 0; r < OTHERS; ++r) {
            const int rr = r < rank ? r : r + 1;  // the other ranks, in order
            v[b][r] = __builtin_bit_cast(f32x4, ld16_coherent_if(in_t(tt), pr, p_off(rr, rg, tt)));
          }
        }
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        if (p0 + b < PAIRS) {
          const int rg = (p0 + b) / NT, tt = (p0 + b) % NT;
          const f32x4 mine = acc[rg][tt];
          // Rank r's partial: this wave's own for r == rank, else the loaded
          // one at index r (below rank) or r - 1 (above).
          auto part_of = [&](int r) -> f32x4 {
            const f32x4 below = v[b][r < OTHERS ? r : OTHERS - 1];
            const f32x4 above = v[b][r > 0 ? r - 1 : 0];
            return r == rank ? mine : (r < rank ? below : above);
          };
          f32x4 tot = part_of(0);
#pragma unroll
          for (int r = 1; r <= OTHERS; ++r) tot += part_of(r);
          store_quad(co, in_t(tt), tot, c_el(rg, tt));
        }
      }
    }
  };
  if (S == 2) {
    reduce.template operator()<PAIRS, 1>();
  } else if (S == 4) {
    reduce.template operator()<(PAIRS < 8 ? PAIRS : 8), 3>();
  } else {
    reduce.template operator()<(NT >= 7 ? 2 : 4), 7>();
  }
  write_stamps();
}

// ---- configurations -------------------------------------------------------

namespace {

template <int NT, int WF>
hipError_t launch_wide_one(const Tactic& t, const GemmParams& p, hipStream_t s) {
  hipLaunchKernelGGL((splitk_wide_kernel<NT, WF>), dim3(t.grid, p.L), dim3(t.threads), t.lds, s, p);
  return hipGetLastError();
}

template <int WF>
hipError_t launch_wide_fmt(const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.nt) {
    case 3: return launch_wide_one<3, WF>(t, p, s);
    case 4: return launch_wide_one<4, WF>(t, p, s);
    case 5: return launch_wide_one<5, WF>(t, p, s);
    case 6: return launch_wide_one<6, WF>(t, p, s);
    case 7: return launch_wide_one<7, WF>(t, p, s);
    case 8: return launch_wide_one<8, WF>(t, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool wide_fits(int T, int N, int ks, int S, int wf, Tactic* t) {
  const bool mx = wf != kBf16;
  const int nt = (T + 15) / 16;
  if (nt < 3 || nt > 8 || N % kWideRows || ks <= 0) return false;
  const int kc = wide_kc(nt, wf);
  if (ks % kc) return false;
  (void)mx;
  t->kind = 3;
  t->nt = nt;
  t->rg = 2;
  t->wk = 1;
  t->wn = kWideWaves;
  t->d = mx ? (nt <= 4 ? 4 : 2) : 4;  // load steps in flight per wave (two per ring slot)
  t->c = 1;
  t->kc = kc;
  t->tile_n = kWideRows;
  t->threads = 64 * kWideWaves;
  t->lds = wide_nbuf(nt, wf) * 16 * nt * kc * 2;
  t->grid = (N / kWideRows) * S;
  t->shape = 0;
  t->fold = 1;
  t->resident = 1;  // 128 KiB of X chunks (or ~200 registers a lane) per workgroup
  (void)S;
  return true;
}

hipError_t launch_wide(const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.wf) {
    case kBf16: return launch_wide_fmt<kBf16>(t, p, s);
    case kMxfp4: return launch_wide_fmt<kMxfp4>(t, p, s);
    case kMxfp8: return launch_wide_fmt<kMxfp8>(t, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace skg
