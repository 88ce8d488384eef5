// Internal interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skg {

// Launch parameters of one split-K GEMM launch over at most 128 token rows.
struct GemmParams {
  const void* w;          // bf16 [N, K], or E2M1 bytes [N, K/2] (MXFP4)
  const uint8_t* wscale;  // E8M0 codes [N, K/32] (MXFP4 only)
  const void* x;          // bf16 [T, K]
  void* c;                // bf16 [T, N]
  float* part;            // FP32 partials [S, T, N] (S > 1)
  uint32_t* cnt;          // arrival counters, one per 16-row group, kCntStride words apart (S > 1)
  int T, N, K, S;
  int ks;       // K / S: the K slice of one split rank
  int kc;       // K elements of X staged in LDS at a time; divides ks
  int nchunks;  // ks / kc
  uint64_t* stamps;  // optional per-workgroup phase stamps
  uint32_t* health;     // owner time-outs: [0] count, [8 + 8r ..] record r (workspace)
  uint32_t owner_wait;  // device-clock ticks (100 MHz) a tile's owner waits for
                        // the other ranks before handing the tile to the last
                        // to arrive (0: hand over at once)
  int pdefer;  // stream kernel: partials held in LDS until the stream ends (1) or
               // stored tile by tile (0)
  // A batch of independent problems of one shape (grid.y = L): problem l
  // reads and writes at these strides from the pointers above.
  int L;
  uint64_t bw, bws, bx, bc;  // bytes between problems: W (or Wq), Wscale, X, C
  uint64_t bpart;            // floats between problems' partials
  uint32_t bcnt;             // counters between problems' counters
  // Output format: 0 bf16 C [T, N]; 1 E4M3FN bytes C [T, N] holding
  // sum * c_scale saturated to +-448 (device/out.h).
  int out_e4m3;
  float c_scale;
  // Persistent kernel's split-K hand-off: 0 arrival counter, 1 tagged
  // mailbox (partials as (value, tag) pairs, 8 bytes per FP32 value; the tag
  // comes from the epoch word at epoch[0], which the last workgroup to start
  // a launch advances; epoch[kCntStride] counts the starts).
  int mailbox;
  uint32_t* epoch;
};

// Choices the library normally makes itself, which tests and tuning runs can
// pin through skgemm_set_override (include/skgemm.h lists their meanings).
// knob() returns the pinned value, or dflt while the knob is unset. Nothing
// else (no environment variable) changes which kernel a call runs.
enum Knob {
  kKnobKind = 0,     // kernel kind: 0 tiled, 1 persistent, 2 cluster, 3 wide
  kKnobStream,       // persistent-kernel shape index
  kKnobShape,        // tiled-kernel shape index
  kKnobFold,         // largest fold of the cluster kernel
  kKnobClusterC,     // 16-byte pieces per lane of bf16 cluster tiles
  kKnobWgPerCu,      // persistent workgroups per CU the grid is sized for
  kKnobPdefer,       // persistent kernel: partials held in LDS (1) or not (0)
  kKnobOwnerWait,    // owner wait bound in device-clock ticks
  kKnobHandoff,      // split-K hand-off of the persistent kernel: 0 counter, 1 mailbox
  kKnobCount
};
int knob(int k, int dflt);

// Words between the split-K arrival counters of two 16-row groups (one
// 128-byte line per counter: the S ranks' arrivals and an owner's polls of
// one tile then meet no other tile's at the device-scope atomic units).
constexpr int kCntStride = 32;

// Health words of a workspace: word 0 counts owner waits that ran out of time
// (the tile then went to the last rank to arrive); words 8 + 8r .. 8 + 8r + 4
// hold the first kHealthRecords of them: {1, first 16-row group of the tile,
// owner rank, problem, ticks waited}.
constexpr int kHealthRecords = 15;
constexpr int kHealthWords = 8 + 8 * kHealthRecords;
// Synchronisation words after the health words of a workspace, one 128-byte
// line each: the chain kernel's grid barrier (a generation, a global count
// and eight group counts), then the mailbox epoch and its start count.
constexpr int kSyncWords = 12 * kCntStride;
// The mailbox epoch words within them (lines 10 and 11).
constexpr int kEpochWord = 10 * kCntStride;

// Records one owner time-out (vector atomics and stores only).
__device__ __forceinline__ void note_timeout(uint32_t* health, uint32_t group, uint32_t rank,
                                             uint32_t waited) {
  if (health == nullptr) return;
  const uint32_t slot = __hip_atomic_fetch_add(health, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (slot < (uint32_t)kHealthRecords) {
    uint32_t* r = health + 8 + 8 * slot;
    r[1] = group;
    r[2] = rank;
    r[3] = blockIdx.y;
    r[4] = waited;
    __hip_atomic_store(r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Moves p's pointers to the problem of this workgroup (blockIdx.y).
__device__ __forceinline__ void select_problem(GemmParams& p) {
  const uint64_t l = blockIdx.y;
  if (l == 0) return;
  p.w = static_cast<const uint8_t*>(p.w) + l * p.bw;
  p.wscale = p.wscale + l * p.bws;
  p.x = static_cast<const uint8_t*>(p.x) + l * p.bx;
  p.c = static_cast<uint8_t*>(p.c) + l * p.bc;
  p.part = p.part + l * p.bpart;
  p.cnt = p.cnt + l * (uint64_t)p.bcnt;
  p.stamps = nullptr;  // stamps describe problem 0 only
}

// A kernel configuration. One workgroup computes a TILE_N x T tile over one K
// slice; its WK * WN waves split that slice WK ways along K (interleaved load
// steps, reduced through LDS in wave order) and the tile WN ways along N;
// each wave owns RG groups of 16 weight rows and keeps D load steps of
// weights in flight per group.
struct Tactic {
  int nt;       // 16-token MFMA tiles: T_pad = 16 * nt, 1..8
  int rg;       // 16-row groups per wave
  int wk;       // waves along K
  int wn;       // waves along N
  int d;        // weight load steps in flight per row group
  int c;        // 16-byte weight pieces per lane per load step (bf16)
  int kc;       // K chunk staged in LDS
  int tile_n;   // 16 * rg * wn
  int threads;  // 64 * wk * wn
  int lds;      // dynamic LDS bytes
  int grid;     // workgroups = (N / tile_n) * split_k
  int wf;       // weight format: 0 bf16, 1 MXFP4, 2 MXFP8 (device/wfmt.h)
  int kind;     // 0: one tile per workgroup; 1: persistent stream kernel;
                // 2: all split ranks of a tile in one workgroup;
                // 3: wide tiles with double-buffered X chunks (33..128 tokens)
  int shape;    // index into the kind's shape table
  int fold;     // kind 2: K windows folded into one MFMA operand (tile rows 16/fold)
  int resident; // workgroups per CU the grid sizing counts on (0: none assumed)
  int pdefer;   // kind 1: partials held in LDS until the stream ends
};

// Picks the configuration for a launch over T <= 128 rows of weight format wf
// (L problems per launch); returns false if no instantiated configuration
// fits (never for validated shapes).
bool pick_tactic(int T, int N, int K, int S, int wf, Tactic* out, int L = 1);

// Whether a launch with this configuration can use the tagged-mailbox
// hand-off: the persistent kernel's deferred and storer organisations
// (not its pipelined epilogue wave), single problems.
bool tactic_mailbox(const Tactic& t);

// Compute units of an MI355X: the grid a launch needs to occupy the chip.
constexpr int kChipCUs = 256;

// Fills the configuration of the one-workgroup-per-tile kernel (kind 2) for a
// launch over T <= 32 rows of L problems, folding at most max_fold ways
// (force_c > 0 pins the pieces per lane for bf16); false if it does not apply.
bool cluster_fits(int T, int N, int ks, int S, int wf, int max_fold, int force_c, Tactic* t, int L = 1);
hipError_t launch_cluster(const Tactic& t, const GemmParams& p, hipStream_t stream);

// Fills the configuration of the wide-tile kernel (kind 3) for 33 <= T <= 128
// rows; false if it does not apply (N % 256, K slice not a whole number of
// X chunks).
bool wide_fits(int T, int N, int ks, int S, int wf, Tactic* t);
hipError_t launch_wide(const Tactic& t, const GemmParams& p, hipStream_t stream);

// Enqueues one launch (T <= 128). Returns the launch's hipError_t.
hipError_t launch_gemm(const Tactic& tac, const GemmParams& p, hipStream_t stream);

// A chain of GEMMs in one cooperative launch (chain.hip): step i multiplies
// A_i [T, dims[i]] (A_0 = x, A_i = c[i-1]) by w[i] [dims[i+1], dims[i]]^T
// into c[i] [T, dims[i+1]], all bf16, split_k = S for every step.
constexpr int kMaxChain = 64;  // SKGEMM_MAX_CHAIN
struct ChainParams {
  const void* w[kMaxChain];
  void* c[kMaxChain];
  const void* x;
  int dims[kMaxChain + 1];
  int fold[kMaxChain];  // per step: K folded 1 or 2 ways (16 / fold rows per tile)
  int L, T, S;
  uint32_t* sync;    // grid barrier words (kSyncWords, one 128-byte line each):
                     // generation, global count, 8 group counts
  uint32_t* health;  // time-out records (workspace health words)
  uint32_t wait_ticks;
};
hipError_t launch_chain(const ChainParams& p, int grid, hipStream_t s);

// Zeros `bytes` (a multiple of 16, 16-byte aligned) with a fill kernel.
hipError_t launch_zero16(void* p, size_t bytes, hipStream_t s);

// Test and helper kernels (bit-exact checks of the device helpers).
hipError_t launch_pack_bf16(const float* in, uint32_t* out, size_t n_pairs, hipStream_t s);
hipError_t launch_pack_e4m3(const float* in, uint32_t* out, size_t n_quads, hipStream_t s);
hipError_t launch_wave_sum(const float* in, float* out, size_t n_waves, hipStream_t s);
hipError_t launch_mxfp4_dequant(const void* wq, const void* ws, void* out, int N, int K,
                                hipStream_t s);
hipError_t launch_mxfp8_dequant(const void* wq, const void* ws, void* out, int N, int K,
                                hipStream_t s);
// Coalesced non-temporal read of `bytes` (a multiple of 16) with
// kReadProbeBlocks workgroups of 512 lanes (four per CU); sink needs
// kReadProbeSinkWords words (workgroup b may write word b % that count).
constexpr int kReadProbeBlocks = 1024;
constexpr int kReadProbeSinkWords = 512;
constexpr uint32_t kReadProbeMagic = 0x9E3779B9u;
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace skg
