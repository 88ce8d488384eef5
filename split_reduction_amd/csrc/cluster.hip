// Split-K GEMM with all split ranks of a tile inside one workgroup.
//
// The pages' kernel keeps the S split ranks of an output tile in one thread
// block cluster: each rank accumulates its contiguous K slice in FP32 and the
// owner sums the ranks' partials in rank order out of distributed shared
// memory (page vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk,
// SplitKGemm.kernel and epilog_warp). On gfx950 the unit that shares on-chip
// memory is the workgroup, so here the workgroup is the cluster: its waves
// form S rank groups of WR = WT / S waves, rank group r streams K slice r, and
// the rank partials meet in LDS. No workspace, no counters, no cross-CU
// traffic: the whole split-K hand-off is one barrier.
//
// Rows per workgroup. One v_mfma_f32_16x16x32_bf16 multiplies 16 A rows by
// 16 B columns. With T <= 16/F tokens, the tile keeps R = 16/F weight rows and
// folds K F ways into the operand: A row f*R + r carries weight row r over
// the f-th K window of the step, B column f*(16/F) + t carries token t over
// the same window, so the F diagonal R x (16/F) blocks of the 16 x 16 result
// are partial sums over disjoint K windows of the same outputs (the other
// blocks pair mismatched windows and are never read). Each loaded weight
// byte still feeds one MFMA row, and small problems spread over F times more
// workgroups. Per rank, a wave's F fold blocks are summed in fold order and
// the rank group's waves in wave order; the rank partials are then summed in
// rank order 0..S-1, rounded to bf16 (RNE) and stored once.
//
// Operands come straight from memory into registers: weights with 16-byte
// buffer loads (C pieces per lane, D steps in flight per wave), and
// activations from X, which every workgroup reads and so stays in L2. Lanes
// of tokens t >= T take an out-of-range offset and read zeros with no memory
// access (page vllm.models.muse_spark.amd.mono.kernels.dev, ld_vec_if).
// MXFP4 lanes load 16 bytes = 32 E2M1 codes = one scale block and decode
// them into four bf16x8 operands (same page, fp4x8_bf16 and e8m0_f32).
// Load layouts: weight loads cover whole 128-byte lines (folded tiles
// natively, unfolded bf16 tiles as row 0-7 / 8-15 line pairs), with the
// non-temporal hint; for folds 1 and 2, activation loads read contiguous runs
// and are moved to their operand lanes with ds_bpermute (block-scaled pieces
// are transposed across lane rows to match). See the notes at each.

#include "device/mfma.h"
#include "device/out.h"
#include "device/pack.h"
#include "device/types.h"
#include "device/wfmt.h"
#include "skgemm_internal.h"

namespace skg {

namespace {

constexpr int kClusterMaxRanks = 8;
constexpr int kClusterMaxWaves = 8;

template <int V>
struct ConstInt {
  static constexpr int value = V;
};

// Load steps kept in flight per wave (operand registers: D * (C + NT*SUBS) * 4).
// Block-scaled weights at one token tile keep 3 (each step also carries four
// activation loads): MXFP4 / MXFP8 T=16 K=7168 N=4096 10.8 -> 10.55 us and
// 13.8 -> 13.3 us against 4, bit-identical; bf16 with one piece keeps 8 in
// eight-wave workgroups (4 or 6 measured slower at T=8 K=7168 N=2048) and 6
// in four-wave ones (8.35 -> 8.28 us there; 12 is slower); bf16 with two
// pieces keeps 2 in folds of 4 and 8 (T=1 K=1024 N=1024 3.37-3.41 -> 3.31 us
// against 4) and 4 below (batches of T=1 K=1024 N=1024: 0.80 against 0.82 us
// a problem with 2).
constexpr int cluster_depth(int nt, int c, bool mx, int f, int wt) {  // mx: block-scaled weights
  return mx ? (nt == 1 ? 3 : 2)
            : (nt == 1 ? (c == 2 ? (f >= 4 ? 2 : 4) : (wt <= 4 ? 6 : 8)) : (c == 2 ? 2 : 4));
}

}  // namespace

// grid = N / R workgroups of 64 * WT threads; workgroup b owns weight rows
// b*R .. b*R + R - 1 over all of K.
template <int NT, int F, int WT, int C, int WF>
__global__ __launch_bounds__(64 * WT) void splitk_cluster_kernel(GemmParams p) {
  select_problem(p);
  constexpr bool MX = WF != kBf16;            // block-scaled weights
  constexpr int LK = lane_k(WF);              // K elements of one lane's 16-byte piece
  constexpr int R = 16 / F;                    // weight rows of the tile
  constexpr int TF = 16 / F;                   // token slots of one fold
  constexpr int LOADS = MX ? 1 : C;            // 16-byte weight loads per lane per step
  constexpr int SUBS = MX ? LK / 8 : C;        // MFMA K-steps per load step
  constexpr int PIECE_K = MX ? 4 * LK : 32 * C;  // K elements of one fold of a step
  constexpr int STEP_K = F * PIECE_K;          // K elements of one load step
  constexpr int SUB_K = MX ? 8 : 32 * F;       // K distance between a lane's sub-steps
  constexpr int D = cluster_depth(NT, C, MX, F, WT);
  // Weight loads in whole 128-byte lines: a fold of F >= 2 already covers
  // 64*F contiguous bytes of each of its R rows per instruction; unfolded
  // bf16 with two pieces loads rows 0-7 and 8-15 as a line pair instead and
  // rearranges at use. Whole-line loads carry the non-temporal hint.
  constexpr bool LINES = F == 1 && !MX && C == 2;
  constexpr int WPOL = (F >= 2 || LINES) ? kPolicyStream : kPolicyDefault;
  static_assert(F == 1 || NT == 1, "folding needs a single token tile");
  static_assert(R >= 2, "outputs are stored in row pairs");

  __shared__ f32x4 red[WT * NT * 64];  // every wave's accumulators
  __shared__ float part[kClusterMaxRanks * 16 * 32];  // rank partials [rank][t][row]

  uint64_t stamp[5];  // optional phase stamps (s_memrealtime, 100 MHz)
  stamp[0] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;   // K block of this lane within an MFMA operand
  const int li = lane & 15;  // A row slot / B column slot of this lane

  const int S = p.S;
  const int T = p.T;
  const int K = p.K;
  const int N = p.N;
  const int WR = WT / S;  // waves per rank group (the host keeps S | WT)
  const int rank = wave / WR;
  const int sub = wave - rank * WR;
  const int n0 = blockIdx.x * R;
  const int kbase = rank * p.ks;
  const int cs = p.ks / STEP_K;                  // load steps of the rank's slice
  const int n_i = (cs - sub + WR - 1) / WR;      // this wave's steps: j = sub + WR * i
  // Every workgroup reads all of X, so workgroups that run side by side on
  // one XCD (every eighth block index under round-robin dispatch) would ask
  // for the same activation lines at the same moment and queue on one L2
  // channel. Each workgroup therefore walks its steps from a different
  // starting point (a rotation; the order inside a rank's slice is free).
  const int rot = n_i > 0 ? (int)((blockIdx.x >> 3) % (unsigned)n_i) : 0;

  const int fa = li / R;   // A: fold of this lane's row slot
  const int ra = li % R;   // A: weight row within the tile
  const int fb = li / TF;  // B: fold of this lane's column slot
  const int tb = li % TF;  // B: token within the fold (F == 1: the token tile's column)

  const uint32_t wrow_bytes = row_bytes(WF, (uint32_t)K);
  const rsrc_t wr = make_rsrc(static_cast<const uint8_t*>(p.w) + (size_t)n0 * wrow_bytes,
                              (uint32_t)R * wrow_bytes);
  const rsrc_t sr = MX ? make_rsrc(p.wscale + (size_t)n0 * (K / 32), (uint32_t)R * (uint32_t)(K / 32))
                       : wr;
  const rsrc_t xr = make_rsrc(p.x, (uint32_t)T * (uint32_t)K * 2u);
  const COut co = make_cout(p);

  // Byte offsets that do not change with the step.
  const uint32_t a_row = LINES ? line_pair_offset(li, 0, wrow_bytes) : (uint32_t)ra * wrow_bytes;
  const uint32_t s_row = (uint32_t)ra * (uint32_t)(K / 32);
  // K offset of a lane's first piece within a step. bf16: piece l of the
  // lane in fold f, K block g covers ((l*F + f)*4 + g)*8 .. +7, so one load
  // instruction covers 64*F contiguous bytes of each row. Block-scaled: the
  // lane's LK codes cover (f*4 + g)*LK .. +LK-1.
  const int a_k = (fa * 4 + g) * (MX ? LK : 8);
  // Activations (bf16). In operand layout neighbouring lanes hold different
  // tokens, so no 4-lane group of a load reads contiguous bytes, and L2 hits
  // move at half the rate of contiguous reads (measured). The loads therefore
  // take contiguous runs (lane m: token m / 4F, 16-byte chunk m % 4F of the
  // token's 64F bytes of the piece) and one ds_bpermute per register moves
  // each lane's chunk to its operand lane (li, g): token li % TF, chunk
  // (li / TF) * 4 + g. Used by folds 1 and 2 (T >= 5 tokens: re-reads as
  // large as the weights); the short launches of folds 4 and 8 gain nothing
  // and lose ~0.3 us to the extra code (measured T=1, K=1024).
  //
  // Block-scaled weights (folds 1 and 2): operand s2 of a lane's 16-byte
  // piece covers elements g*LK + 8*s2 of the step window, so the activation
  // operand s2 of the four lane rows would be four runs LK elements apart.
  // The weight pieces are therefore transposed across the lane rows at use
  // (transpose_pieces: operand s2 of lane row g becomes elements 32*s2 + 8*g),
  // and activation load s2 takes, for each (token, fold) slot li', the 64
  // contiguous bytes 32*s2 .. 32*s2 + 31 of its window (lane 4*li' + q takes
  // the q-th 16 bytes); operand lane (li, g) reads load lane 4*li + g.
  constexpr bool xperm = !MX && F <= 2;
  constexpr bool MXT = MX && F <= 2;
  constexpr int XSUB_K = MXT ? 32 : SUB_K;  // K distance between a lane's activation loads
  const int xs = lane >> 2;                 // MXT: (token, fold) slot of this lane's load
  const int xt = xperm ? lane / (4 * F) : (MXT ? xs % TF : tb);   // token of this lane's load
  const int b_k = xperm ? (lane % (4 * F)) * 8
                        : (MXT ? (xs / TF) * 4 * LK + 8 * (lane & 3) : (fb * 4 + g) * (MX ? LK : 8));
  const int b_src = xperm ? 4 * ((li % TF) * 4 * F + (li / TF) * 4 + g)  // bpermute byte address
                          : 4 * (4 * li + g);
  bool b_ok[NT];
  uint32_t b_row[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int t = tt * 16 + xt;
    b_ok[tt] = t < T;
    b_row[tt] = (uint32_t)(b_ok[tt] ? t : 0) * (uint32_t)K * 2u;
  }
  auto x_operand = [&](u32x4 v) -> bf16x8 {
    if constexpr (xperm || MXT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(b_src, (int)v[e]);
    }
    return as_bf16x8(v);
  };

  u32x4 ra_ring[D][LOADS];
  uint32_t sc_ring[D];
  u32x4 rb_ring[D][NT][SUBS];
  auto issue = [&](int slot, int i) {
    const bool ok = i < n_i;
    int ir = i + rot;
    if (ir >= n_i) ir -= n_i;
    const int kel = kbase + (sub + WR * ir) * STEP_K;
    // Line pairs: window li / 8 sits in a_row, so the lane's K block is g.
    const uint32_t a_off = elem_byte(WF, (uint32_t)(kel + (LINES ? 8 * g : a_k)));
#pragma unroll
    for (int l = 0; l < LOADS; ++l)
      ra_ring[slot][l] = ld16_if<WPOL>(ok, wr, a_row + a_off + (LINES ? 8u * wrow_bytes : (uint32_t)(2 * SUB_K)) * l);
    if constexpr (MXT) {
      // The scales of the lane's window (4*LK / 32 bytes): after the
      // transpose, operand s2 lies in the window's block s2.
      const uint32_t so = s_row + (uint32_t)((kel + fa * 4 * LK) / 32);
      sc_ring[slot] = WF == kMxfp4 ? ld4_if(ok, sr, so) : ld2_if(ok, sr, so);
    } else if constexpr (MX) {
      sc_ring[slot] = ld1_if(ok, sr, s_row + (uint32_t)((kel + a_k) / 32));
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int s2 = 0; s2 < SUBS; ++s2)
        rb_ring[slot][tt][s2] =
            ld16_if(ok && b_ok[tt], xr, b_row[tt] + (uint32_t)(kel + b_k + XSUB_K * s2) * 2u);
  };

  f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    u32x4 a[LOADS];
    if constexpr (LINES) {
      line_pair_to_operands(ra_ring[slot][0], ra_ring[slot][1], a[0], a[1]);
    } else if constexpr (MXT) {
      a[0] = transpose_pieces<WF>(ra_ring[slot][0]);
    } else {
#pragma unroll
      for (int l = 0; l < LOADS; ++l) a[l] = ra_ring[slot][l];
    }
#pragma unroll
    for (int s2 = 0; s2 < SUBS; ++s2) {
      bf16x8 af;
      if constexpr (MX) {
        af = decode_operand<WF>(a[0], s2, e8m0_f32(MXT ? (sc_ring[slot] >> (8 * s2)) & 0xFFu : sc_ring[slot]));
      } else {
        af = as_bf16x8(a[s2]);
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma_bf16(af, x_operand(rb_ring[slot][tt][s2]), acc[tt]);
    }
  };

#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, s);
  stamp[1] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  int q = 0;
  for (; q + D <= n_i; q += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      compute(s);
      issue(s, q + D + s);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (q + s < n_i) compute(s);

  stamp[2] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;

  // ---- the hand-off: every wave's accumulators into LDS --------------------
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) red[(wave * NT + tt) * 64 + lane] = acc[tt];
  __syncthreads();
  stamp[3] = p.stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const float* redf = reinterpret_cast<const float*>(red);

  // Pass 1: rank partial of (rank, token, row pair) = its waves' fold blocks,
  // folds in order within a wave, waves in order. Pass 2: rank-order sum, one
  // RNE rounding, one store per row pair. The split (S, hence waves per rank)
  // is dispatched once to compile-time loop bounds, so both passes unroll.
  constexpr int PAIRS = R / 2;
  const int per_rank = PAIRS * T;
  // Folds 4 and 8 (T <= 4, short launches): runtime bounds keep the
  // registers of the many fold blocks in check.
  auto reduce_rt = [&]() {
    for (int o = tid; o < S * per_rank; o += 64 * WT) {
      const int rk = o / per_rank;
      const int rem = o - rk * per_rank;
      const int t = rem / PAIRS;
      const int r = (rem - t * PAIRS) * 2;
      const int tt = t / 16;
      const int tl = t - tt * 16;
      float v0 = 0.f, v1 = 0.f;
      for (int s2 = 0; s2 < WR; ++s2) {
        const float* wbase = redf + (size_t)(((rk * WR + s2) * NT + tt) * 64) * 4;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int row = f * R + r;
          const int col = f * TF + tl;
          const float* e = wbase + (16 * (row >> 2) + col) * 4 + (row & 3);
          v0 += e[0];
          v1 += e[1];
        }
      }
      part[(rk * 32 + t) * 16 + r] = v0;
      part[(rk * 32 + t) * 16 + r + 1] = v1;
    }
    __syncthreads();
    for (int o = tid; o < per_rank; o += 64 * WT) {
      const int t = o / PAIRS;
      const int r = (o - t * PAIRS) * 2;
      float v0 = part[t * 16 + r];
      float v1 = part[t * 16 + r + 1];
      for (int rk = 1; rk < S; ++rk) {
        v0 += part[(rk * 32 + t) * 16 + r];
        v1 += part[(rk * 32 + t) * 16 + r + 1];
      }
      store_pair(co, true, v0, v1, (uint32_t)t * (uint32_t)N + (uint32_t)(n0 + r));
    }
  };
  auto reduce = [&](auto s_c) {
    constexpr int SC = decltype(s_c)::value;
    constexpr int WRC = WT / SC;
    for (int o = tid; o < SC * per_rank; o += 64 * WT) {
      const int rk = o / per_rank;
      const int rem = o - rk * per_rank;
      const int t = rem / PAIRS;
      const int r = (rem - t * PAIRS) * 2;
      const int tt = t / 16;
      const int tl = t - tt * 16;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < WRC; ++s2) {
        const float* wbase = redf + (size_t)(((rk * WRC + s2) * NT + tt) * 64) * 4;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int row = f * R + r;  // rows row, row + 1 sit in one lane (R even)
          const int col = f * TF + tl;
          const float* e = wbase + (16 * (row >> 2) + col) * 4 + (row & 3);
          v0 += e[0];
          v1 += e[1];
        }
      }
      part[(rk * 32 + t) * 16 + r] = v0;
      part[(rk * 32 + t) * 16 + r + 1] = v1;
    }
    __syncthreads();
    for (int o = tid; o < per_rank; o += 64 * WT) {
      const int t = o / PAIRS;
      const int r = (o - t * PAIRS) * 2;
      float v0 = part[t * 16 + r];
      float v1 = part[t * 16 + r + 1];
#pragma unroll
      for (int rk = 1; rk < SC; ++rk) {
        v0 += part[(rk * 32 + t) * 16 + r];
        v1 += part[(rk * 32 + t) * 16 + r + 1];
      }
      store_pair(co, true, v0, v1, (uint32_t)t * (uint32_t)N + (uint32_t)(n0 + r));
    }
  };
  if constexpr (F <= 2) {
    switch (S) {  // S divides WT (the host keeps S | WT), S <= 8
      case 1: reduce(ConstInt<1>{}); break;
      case 2: reduce(ConstInt<(WT >= 2 ? 2 : 1)>{}); break;
      case 4: reduce(ConstInt<(WT >= 4 ? 4 : 1)>{}); break;
      default: reduce(ConstInt<(WT >= 8 ? 8 : 1)>{}); break;
    }
  } else {
    reduce_rt();
  }
  // Thread 0 writes the stamps (vector stores): entry, loads issued, wave 0's
  // stream done, all waves' sums in LDS, exit.
  if (p.stamps != nullptr && tid == 0) {
    stamp[4] = __builtin_amdgcn_s_memrealtime();
    const rsrc_t sr8 = make_rsrc(p.stamps + (size_t)blockIdx.x * 8, 64);
#pragma unroll
    for (int i = 0; i < 5; ++i)
      st8_if(true, u32x2{(uint32_t)stamp[i], (uint32_t)(stamp[i] >> 32)}, sr8, 8u * i);
  }
}

// ---- configurations ---------------------------------------------------------

namespace {

template <int NT, int F, int WT, int C, int WF>
hipError_t launch_cluster_one(const Tactic& t, const GemmParams& p, hipStream_t s) {
  hipLaunchKernelGGL((splitk_cluster_kernel<NT, F, WT, C, WF>), dim3(t.grid, p.L), dim3(t.threads), 0, s, p);
  return hipGetLastError();
}

template <int NT, int F, int C, int WF>
hipError_t launch_cluster_wt(const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.wk) {
    case 4: return launch_cluster_one<NT, F, 4, C, WF>(t, p, s);
    case 8: return launch_cluster_one<NT, F, 8, C, WF>(t, p, s);
  }
  return hipErrorInvalidValue;
}

template <int C, int WF>
hipError_t launch_cluster_f(const Tactic& t, const GemmParams& p, hipStream_t s) {
  if (t.nt == 2) return t.fold == 1 ? launch_cluster_wt<2, 1, C, WF>(t, p, s) : hipErrorInvalidValue;
  if (t.nt != 1) return hipErrorInvalidValue;
  switch (t.fold) {
    case 1: return launch_cluster_wt<1, 1, C, WF>(t, p, s);
    case 2: return launch_cluster_wt<1, 2, C, WF>(t, p, s);
    case 4: return launch_cluster_wt<1, 4, C, WF>(t, p, s);
    case 8: return launch_cluster_wt<1, 8, C, WF>(t, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool cluster_fits(int T, int N, int ks, int S, int wf, int max_fold, int force_c, Tactic* t, int L) {
  const bool mx = wf != kBf16;
  if (T < 1 || T > 32 || S > kClusterMaxRanks || ks <= 0) return false;
  const int nt = (T + 15) / 16;
  // Widest fold whose token slots still hold every token.
  int fold = 1;
  if (nt == 1) {
    int tp = 1;
    while (tp < T) tp *= 2;
    fold = 16 / tp;
    if (fold > 8) fold = 8;
  }
  // Taller tiles while the grid still covers every CU: each workgroup reads
  // all of X, so halving the fold halves the X re-reads (measured T=8,
  // K=7168, N=4096: 16-row tiles 16.3 us, 8-row tiles 21.8 us).
  while (fold > 1 && (long)(N / (32 / fold)) * L >= kChipCUs) fold /= 2;
  if (fold > max_fold) fold = max_fold;
  // Pieces per lane (bf16): two unless the tile is folded and its rank
  // slices hold at least 64 / S one-piece steps each (S * steps >= 64;
  // measured K=7168, S=4, T=5..8: 7.7-9.8 us with one piece against
  // 8.3-10.6 us with two; K=2048, S=2 (32 steps): 5.9 against 5.5 us).
  // Unfolded tiles keep two, which their whole-line load pairs need.
  int c_first = 2;
  if (!mx && fold >= 2 && ks % (fold * 32) == 0 && S * (ks / (fold * 32)) >= 64) c_first = 1;
  for (int ci = 0; ci < 2; ++ci) {
    const int c = ci == 0 ? c_first : 3 - c_first;
    if (mx && c == 2) continue;  // one 16-byte MXFP4 piece is a whole step
    if (force_c > 0 && !mx && c != force_c) continue;
    for (int f = fold; f >= 1; f /= 2) {
      const int step = f * (mx ? 4 * lane_k(wf) : 32 * c);
      if (ks % step) continue;
      const int cs = ks / step;
      // Waves: a power of two in 4..8, at least S (so S divides it), and
      // no more per rank group than the slice has steps. Eight waves with
      // twice the steps each beat sixteen (measured T=16 K=7168 N=4096:
      // MXFP4 11.7 -> 10.8 us, MXFP8 14.6 -> 14.1 us; bf16 T=8: 8.45 ->
      // 8.37 us at N=2048, 13.7 -> 13.5 us at N=4096). A single bf16 problem
      // runs faster still on four (one box, three runs each: T=8 K=7168
      // N=2048 8.49 -> 8.36 us, T=2 K=4096 N=4096 8.84 -> 8.06 us, T=4..16
      // K=7168 N=2048..4096 1-2 % faster); block-scaled weights do not
      // (MXFP8 13.25 -> 13.76 us) and neither do batches (T=8 K=7168 N=2048,
      // L=8: 5.79 -> 6.02 us a problem), so they keep eight. The cap never
      // goes below S (each rank group needs a wave).
      const int cap = (wf != kBf16 || L > 1 || S > 4) ? kClusterMaxWaves : 4;
      const int want = S * cs < cap ? S * cs : cap;
      int wt = 4;
      while (wt < want) wt *= 2;
      if (wt < S) continue;
      if (N % (16 / f)) continue;
      t->kind = 2;
      t->nt = nt;
      t->fold = f;
      t->rg = 1;
      t->wk = wt;
      t->wn = 1;
      t->d = cluster_depth(nt, c, mx, f, wt);
      t->c = c;
      t->kc = ks;
      t->tile_n = 16 / f;
      t->threads = 64 * wt;
      t->lds = 0;
      t->grid = N / (16 / f);
      t->shape = 0;
      return true;
    }
  }
  return false;
}

hipError_t launch_cluster(const Tactic& t, const GemmParams& p, hipStream_t s) {
  switch (t.wf) {
    case kMxfp4: return launch_cluster_f<1, kMxfp4>(t, p, s);
    case kMxfp8: return launch_cluster_f<1, kMxfp8>(t, p, s);
  }
  return t.c == 2 ? launch_cluster_f<2, kBf16>(t, p, s) : launch_cluster_f<1, kBf16>(t, p, s);
}

}  // namespace skg
