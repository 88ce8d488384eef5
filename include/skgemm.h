/*
 * skgemm -- split-K decode GEMM for AMD MI355X (gfx950, CDNA4).
 *
 * C ABI of libskgemm.so. Plain pointers and sizes only; every pointer passed
 * to a compute entry point is DEVICE memory owned by the caller (for example
 * the storage of a torch tensor). The library never frees, reallocates or
 * synchronises caller memory. Work is enqueued on the caller's stream and
 * nothing is synchronised on return, as with the graph-compatible launch
 * wrapper on page vllm.models.common.ops.moe_tail_fusion.primitives
 * (CUDAGraphCompatibleWrapper: launch on the current stream, no producer
 * sync).
 *
 * The operation (page
 * vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk, module
 * summary and SplitKGemm): C[T, N] = X[T, K] . W[N, K]^T. Each of split_k
 * contiguous, equal K slices is accumulated in FP32; the slices' partials are
 * reduced once in slice order, rounded to bf16 (round to nearest even) and C
 * is stored once. The weights take the MFMA's row operand ("kernel-M carries
 * public N").
 *
 * Layouts (row-major, the last index contiguous):
 *   W      bf16  [N, K]     (K contiguous; SplitKGemm.kernel: A is K-major)
 *   X      bf16  [T, K]     (K contiguous; B is K-major)
 *   C      bf16  [T, N]     (N contiguous)
 *   Wq     uint8 [N, K/2]   two E2M1 codes per byte: element k of a row is in
 *                           byte k/2, the low nibble when k is even (page
 *                           vllm.models.muse_spark.amd.mono.kernels.dev,
 *                           fp4x8_bf16: a dword of 8 E2M1, low nibble first)
 *   Wscale uint8 [N, K/32]  one E8M0 code per 32-element K block; code c
 *                           stands for 2^(c-127) (same page, e8m0_f32).
 *                           Codes must lie in 1..254.
 *
 * Return codes: 0 on success, a negative SKGEMM_E* code otherwise. When an
 * argument check fails nothing is enqueued and C is untouched. Faults of the
 * enqueued work surface asynchronously on the caller's stream.
 *
 * Concurrency: calls on one stream are ordered by the stream. Each
 * (device, stream) pair owns its own split-K workspace, so calls on different
 * streams do not share partial buffers.
 */
#ifndef SKGEMM_H
#define SKGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* HIP's own stream handle type */

#define SKGEMM_API __attribute__((visibility("default")))

enum skgemm_status {
  SKGEMM_OK = 0,
  SKGEMM_EINVAL = -1, /* null pointer, negative size, split_k not in {1,2,4,8} */
  SKGEMM_EALIGN = -2, /* a pointer is not 16-byte aligned                      */
  SKGEMM_ESHAPE = -3, /* N % 16, K % (32*split_k) (bf16) or K % (128*split_k)
                         (MXFP4) non-zero, or a size above the limits below   */
  SKGEMM_ENOMEM = -4, /* split-K workspace could not be allocated, or it would
                         have to grow while the stream is being captured      */
  SKGEMM_EHIP = -5,   /* a HIP runtime call failed; see skgemm_last_hip_error */
  SKGEMM_ESCRATCH = -6 /* skgemm_bf16_noalloc: the call needs more split-K
                          partials than its fixed scratch holds              */
};

/* Size limits (checked; SKGEMM_ESHAPE beyond them). T has no upper limit:
 * token counts above 128 are processed in blocks of 128 rows. */
#define SKGEMM_MAX_N (1 << 18)
#define SKGEMM_MAX_K (1 << 22)
#define SKGEMM_MAX_BATCH 4096

/*
 * skgemm_bf16: C = X . W^T with bf16 W, X, C and FP32 accumulation.
 *   W, X, C  device pointers, 16-byte aligned, layouts above.
 *   T >= 0   tokens (rows of X and C). T == 0 or N == 0 enqueues nothing.
 *   N >= 0   output features, N % 16 == 0.
 *   K >= 0   reduction length, K % (32 * split_k) == 0. K == 0 stores zeros.
 *   split_k  1, 2, 4 or 8: number of contiguous K slices, slice r covering
 *            [r*K/split_k, (r+1)*K/split_k) (SplitKGemm.kernel splits K evenly
 *            over the cluster ranks; shapes are validated, never padded).
 *   stream   HIP stream to enqueue on (0 = the null stream).
 * With split_k > 1 the first call on a stream allocates that stream's
 * workspace (see skgemm_reserve) unless one large enough exists.
 */
SKGEMM_API int skgemm_bf16(const void* W, const void* X, void* C, int T, int N, int K,
                           int split_k, hipStream_t stream);

/*
 * skgemm_bf16_e4m3: skgemm_bf16 with an 8-bit output: C8[t, n] is the OCP
 * E4M3FN code of min(max(sum * c_scale, -448), 448), rounded to nearest even,
 * where sum is the same FP32 rank-order sum skgemm_bf16 rounds to bf16 (the
 * E4M3 packing of page vllm.models.deepseek_v41.amd.mono.common.ops,
 * fp8_pack4, on values brought into its range by the scale and a
 * saturation). The product with c_scale is one FP32 multiply.
 *   C8       uint8 [T, N] row-major, device memory, 16-byte aligned.
 *   c_scale  finite and > 0 (SKGEMM_EINVAL otherwise); typically 448 over
 *            the largest |C| expected, or a power of two.
 *   Other arguments, limits and errors as skgemm_bf16. Non-finite sums are
 *   outside the contract.
 */
SKGEMM_API int skgemm_bf16_e4m3(const void* W, const void* X, void* C8, float c_scale, int T, int N,
                                int K, int split_k, hipStream_t stream);

/*
 * skgemm_bf16_chain: L dependent GEMMs in one launch, the output of each the
 * activations of the next: step i computes C[i][T, dims[i+1]] =
 * A_i . W[i]^T with A_0 = X and A_i = C[i-1], each step as skgemm_bf16 would
 * (split_k contiguous K slices in FP32, rank-order sum, bf16 RNE, stored
 * once). This is the launch overlap of page
 * vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk
 * (SplitKGemm.__call__ with use_pdl: the weight loads of the next kernel go
 * out before it waits for its predecessor, the activation loads after): the
 * weights of step i+1 are loaded while step i finishes, and only the
 * activation loads wait for C[i] (a grid-wide barrier between steps).
 *   W, C     host arrays of L device pointers: W[i] bf16 [dims[i+1], dims[i]],
 *            C[i] bf16 [T, dims[i+1]], 16-byte aligned; C[i] must not
 *            overlap its input (X for i = 0, else C[i-1]) (SKGEMM_EINVAL).
 *   X        bf16 [T, dims[0]], device memory, 16-byte aligned.
 *   dims     host array of L + 1 sizes, each >= 1 and within the size limits.
 *   1 <= L <= SKGEMM_MAX_CHAIN, 1 <= T <= 16, split_k in {1, 2, 4, 8}.
 *   Shapes: dims[i] % (32 * split_k) == 0 for i < L and dims[i] % 16 == 0
 *   for i >= 1 (SKGEMM_ESHAPE).
 * The launch is cooperative (all workgroups resident at once, one per CU);
 * it uses the stream's workspace for its barrier words, so chains on one
 * stream are ordered and chains on different streams do not share them. A
 * barrier wait that runs out (not expected: the launch is cooperative) is
 * recorded in skgemm_health as a record with tile group 0xFFFFFFFF and the
 * step as its rank.
 */
#define SKGEMM_MAX_CHAIN 64
SKGEMM_API int skgemm_bf16_chain(const void* const* W, const void* X, void* const* C, const int* dims,
                                 int L, int T, int split_k, hipStream_t stream);

/*
 * skgemm_bf16_noalloc: skgemm_bf16 for callers that cannot allocate device
 * memory -- code under HIP graph capture without a prior skgemm_reserve,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * kernels and results (bit for bit) as skgemm_bf16, but the split-K
 * partials and counters live in a fixed scratch array of
 * SKGEMM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; this call never allocates or frees memory.
 *   Limit: with split_k > 1, split_k * min(T, 128) * N * 4 bytes of partials
 *   must fit in SKGEMM_NOALLOC_SCRATCH_BYTES - SKGEMM_NOALLOC_PART_OFFSET
 *   (39.8 MB: e.g. T = 128, N = 16384 at split_k = 4); larger calls return
 *   SKGEMM_ESCRATCH before any device work. split_k = 1 needs no scratch.
 *   Every call on one GPU shares that GPU's scratch, from any stream: calls
 *   that may overlap in time (other streams, other threads) race and give
 *   wrong results; order them (one stream, or events). The counter area is
 *   cleared on the device's first calls (a fill kernel enqueued on `stream`;
 *   inside a graph capture the clear is captured too) and every call leaves
 *   it zeroed. Time-outs of the bounded owner wait are not reported by
 *   skgemm_health for this entry point.
 */
#define SKGEMM_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
#define SKGEMM_NOALLOC_PART_OFFSET ((size_t)(2 << 20) + 4096)
SKGEMM_API int skgemm_bf16_noalloc(const void* W, const void* X, void* C, int T, int N, int K,
                                   int split_k, hipStream_t stream);

/*
 * skgemm_mxfp4: C = X . dequant(Wq, Wscale)^T. The weights are decoded exactly
 * to bf16 in registers (E2M1 value times 2^(code-127)), then multiplied as in
 * skgemm_bf16 (page vllm.models.muse_spark.amd.mono.kernels.dev, fp4x8_bf16).
 *   Wq, X, C 16-byte aligned; Wscale needs no alignment.
 *   K % (128 * split_k) == 0 (each lane decodes 32 consecutive K elements,
 *   one whole scale block, per 16-byte load). Other arguments as skgemm_bf16.
 */
SKGEMM_API int skgemm_mxfp4(const void* Wq, const void* Wscale, const void* X, void* C, int T,
                            int N, int K, int split_k, hipStream_t stream);

/*
 * skgemm_mxfp8: C = X . dequant(Wq8, Wscale)^T with MXFP8 weights: one OCP
 * E4M3FN code per byte, Wq8 uint8 [N, K] row-major (element k of a row in
 * byte k), and one E8M0 scale code per 32-element K block, Wscale uint8
 * [N, K/32]. w[n, k] = E4M3(code) * 2^(scale - 127), decoded exactly to bf16
 * in registers (v_cvt_scalef32_pk_bf16_fp8) and multiplied as in skgemm_bf16:
 * the block scaling of skgemm_mxfp4 (page
 * vllm.models.muse_spark.amd.mono.kernels.dev, e8m0_f32) with the E4M3
 * elements of page vllm.models.deepseek_v41.amd.mono.common.ops, fp8_pack4.
 *   Wq8, X, C 16-byte aligned; Wscale needs no alignment.
 *   K % (64 * split_k) == 0 (each lane decodes 16 consecutive K elements,
 *   half a scale block, per 16-byte load). Other arguments as skgemm_bf16.
 */
SKGEMM_API int skgemm_mxfp8(const void* Wq8, const void* Wscale, const void* X, void* C, int T,
                            int N, int K, int split_k, hipStream_t stream);

/*
 * skgemm_bf16_batched, skgemm_mxfp4_batched, skgemm_mxfp8_batched: L
 * independent problems of one
 * shape in one launch (the pages' batch dimension L: SplitKGemm.kernel takes
 * A (M,K,L), B (N,K,L), C (M,N,L) and SplitKGemm.__call__ launches the L
 * problems as the third grid dimension). Problem l reads W + l*w_stride, X + l*x_stride (and Wscale +
 * l*wscale_stride) and writes C + l*c_stride; strides are in bytes. Each
 * problem is computed exactly as the single call with the same arguments
 * would compute it, and one launch amortises the dispatch cost over L.
 *   1 <= L <= SKGEMM_MAX_BATCH. For L > 1: w/wq, x and c strides are
 *   multiples of 16 (every problem's operands stay 16-byte aligned); a zero
 *   W or X stride shares that operand across the batch; c_stride >= T*N*2 so
 *   outputs do not overlap (SKGEMM_EINVAL otherwise; SKGEMM_EALIGN for a
 *   misaligned stride). Other arguments as skgemm_bf16 / skgemm_mxfp4; with
 *   split_k > 1 the workspace holds L problems (skgemm_reserve_batched).
 */
SKGEMM_API int skgemm_bf16_batched(const void* W, const void* X, void* C, int T, int N, int K,
                                   int split_k, int L, size_t w_stride, size_t x_stride,
                                   size_t c_stride, hipStream_t stream);
SKGEMM_API int skgemm_mxfp4_batched(const void* Wq, const void* Wscale, const void* X, void* C,
                                    int T, int N, int K, int split_k, int L, size_t wq_stride,
                                    size_t wscale_stride, size_t x_stride, size_t c_stride,
                                    hipStream_t stream);
SKGEMM_API int skgemm_mxfp8_batched(const void* Wq8, const void* Wscale, const void* X, void* C,
                                    int T, int N, int K, int split_k, int L, size_t wq8_stride,
                                    size_t wscale_stride, size_t x_stride, size_t c_stride,
                                    hipStream_t stream);

/*
 * skgemm_reserve: make sure the workspace of (current device, stream) can
 * serve any call with T <= max_T (capped at 128, the block size), N <= max_N
 * and split_k <= max_split_k. Call it before capturing a stream into a HIP
 * graph: inside a capture the workspace can not grow (SKGEMM_ENOMEM). The
 * workspace is FP32 partials [split_k, min(T,128), N] and one uint32 counter
 * per 16 output rows, each on a 128-byte line of its own; counters return to
 * zero at the end of every call.
 * Workspace lifetime: a workspace that has to grow is replaced by a new,
 * larger one; the old one is not freed but kept until skgemm_release, because
 * a graph captured while it was current still uses it on every replay. So a
 * graph may be captured after skgemm_reserve and replayed after later eager
 * calls of any size on the same stream. skgemm_release frees every
 * workspace: graphs that use one must not be replayed after it.
 */
SKGEMM_API int skgemm_reserve(int max_T, int max_N, int max_split_k, hipStream_t stream);

/*
 * skgemm_reserve_batched: skgemm_reserve for batched calls of up to max_L
 * problems (1 <= max_L <= SKGEMM_MAX_BATCH); skgemm_reserve is max_L = 1.
 */
SKGEMM_API int skgemm_reserve_batched(int max_T, int max_N, int max_split_k, int max_L,
                                      hipStream_t stream);

/* skgemm_release: free every workspace of the calling process. Synchronises
 * each workspace's device first and restores the calling thread's current
 * device afterwards. Not to be called while other threads enqueue work. */
SKGEMM_API int skgemm_release(void);

/*
 * skgemm_mxfp4_dequant: W_out bf16 [N, K] = E2M1(Wq) * 2^(Wscale - 127),
 * elementwise, exact (the decode the GEMM applies in registers; exported for
 * bit-exact testing). K % 32 == 0, Wq and W_out 16-byte aligned.
 */
SKGEMM_API int skgemm_mxfp4_dequant(const void* Wq, const void* Wscale, void* W_out, int N, int K,
                                    hipStream_t stream);

/*
 * skgemm_mxfp8_dequant: W_out bf16 [N, K] = E4M3(Wq8) * 2^(Wscale - 127),
 * the in-register decode of skgemm_mxfp8 on its own (bit-exact tests).
 * Exact for scale codes 10..246 (every product then normal and finite in
 * bf16); codes 0x7F and 0xFF give NaN. K % 32 == 0; Wq8 and W_out 16-byte
 * aligned.
 */
SKGEMM_API int skgemm_mxfp8_dequant(const void* Wq8, const void* Wscale, void* W_out, int N, int K,
                                    hipStream_t stream);

/*
 * skgemm_pack_bf16: out[i] = bf16(in[2i]) | bf16(in[2i+1]) << 16, round to
 * nearest even, the epilogue's packing (page
 * vllm.models.muse_spark.amd.mono.kernels.dev, bf16_pair). in: float
 * [2*n_pairs], out: uint32 [n_pairs], device memory, 16-byte aligned.
 */
SKGEMM_API int skgemm_pack_bf16(const float* in, uint32_t* out, size_t n_pairs, hipStream_t stream);

/*
 * skgemm_pack_e4m3: out[i] = four OCP E4M3FN bytes of in[4i..4i+3], the first
 * in the low byte, round to nearest even; inputs must satisfy |x| <= 448
 * (page vllm.models.deepseek_v41.amd.mono.common.ops, fp8_pack4: "already in
 * range"). in: float [4*n_quads], out: uint32 [n_quads], 16-byte aligned.
 */
SKGEMM_API int skgemm_pack_e4m3(const float* in, uint32_t* out, size_t n_quads, hipStream_t stream);

/*
 * skgemm_wave_sum: for each group of 64 floats, every lane of one wavefront
 * ends with the butterfly sum over lane offsets 32, 16, 8, 4, 2, 1 in that
 * order, each step value[i] + value[i ^ off] in FP32 (page
 * vllm.models.deepseek_v41.amd.mono.common.ops, butterfly / xred / xshfl:
 * the order is the numerical contract; 32 and 16 go through
 * v_permlane32/16_swap, the rest through DPP). in, out: float [64*n_waves].
 */
SKGEMM_API int skgemm_wave_sum(const float* in, float* out, size_t n_waves, hipStream_t stream);

/*
 * skgemm_health: the bounded-wait report of (current device, stream) (page
 * vllm.models.muse_spark.amd.mono.kernels.dev, _spin_bounded: a time-out
 * writes a record instead of hanging). With split_k > 1 the owner rank of a
 * tile waits a bounded time for the other ranks; when that time runs out it
 * hands the tile to the last rank to arrive (the result is unchanged) and
 * records it. Copies min(n_words, 128) words to host memory `words` and
 * clears them on the device: word 0 = time-outs since the last call; words
 * 8 + 8r .. 8 + 8r + 4 (r < min(count, 15)) = {1, the tile's first 16-row
 * group, owner rank, problem index in a batch, ticks waited}; other words 0.
 * A time-out means the launch's workgroups were not all resident at once
 * (e.g. a concurrent kernel held CUs): a slow path, not a wrong result.
 * Synchronises `stream`; SKGEMM_EINVAL under graph capture. A stream with no
 * workspace yet reports zeros.
 */
SKGEMM_API int skgemm_health(uint32_t* words, size_t n_words, hipStream_t stream);

/*
 * skgemm_read_probe: a reference for the weight stream, not part of the
 * method: reads `bytes` of device memory at src once, with coalesced 16-byte
 * non-temporal loads, 1024 workgroups of 512 lanes each reading one
 * contiguous block (the fastest streaming read measured on the chip), and
 * computes nothing from them. The time it takes is the
 * streaming-read rate the GEMM kernels are compared with at the same byte
 * count. src: 16-byte aligned, bytes a multiple of 16. sink: device memory for
 * 512 uint32 words, which the probe does not normally write. Returns
 * SKGEMM_EINVAL for a null pointer or a bad size, SKGEMM_EALIGN for
 * misaligned pointers.
 */
SKGEMM_API int skgemm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * skgemm_tactic_for: describe, as a short JSON object written to buf
 * (NUL-terminated, truncated to buf_len), the kernel configuration a call with
 * these sizes would launch. weight_format: 0 bf16 (skgemm_bf16), 1 MXFP4
 * (skgemm_mxfp4), 2 MXFP8 (skgemm_mxfp8); SKGEMM_EINVAL for others. Returns
 * the same code the compute call's argument checks would (pointers excluded).
 * Host only; touches no device.
 */
SKGEMM_API int skgemm_tactic_for(int T, int N, int K, int split_k, int weight_format, char* buf,
                                 size_t buf_len);

/*
 * skgemm_set_timeline: opt-in phase stamps of the persistent stream kernel
 * (page vllm.models.deepseek_v41.amd.mono.common.ops, module note and
 * memrealtime: timeline phase stamps from s_memrealtime, the 100 MHz device
 * clock). While set, every workgroup w of a stream-kernel launch writes
 * uint64 clock values to buf[8*w .. 8*w+7]: kernel entry, X staged in LDS,
 * weight stream done, own partial stores complete, exit, then (counter
 * hand-off, as its wave 0 sees it; 0 elsewhere) arrivals done and the owned
 * tiles' polls done, and 0. The cluster kernel writes entry, first loads
 * issued, wave 0's stream done, every wave's sums in LDS, exit; the wide
 * kernel entry, first X chunk staged, stream done, its column's partial
 * stored, exit. Device memory,
 * caller-owned, 8-byte aligned; `capacity` is its length in uint64. Launches
 * whose grid needs more than capacity/8 workgroups write nothing. Pass
 * buf = NULL to turn stamping off (the default). Process-wide setting.
 */
SKGEMM_API int skgemm_set_timeline(void* buf, size_t capacity);

/*
 * skgemm_set_override: pins a choice the library normally makes itself; for
 * tests and tuning runs, not needed in normal use (nothing else, no
 * environment variable, changes which kernel a call runs). value -1 restores
 * the library's own choice; other negative values and unknown knobs give
 * SKGEMM_EINVAL. Process-wide, read by every later call and by
 * skgemm_tactic_for; a pinned kernel kind or shape that cannot take a call's
 * sizes makes that call return SKGEMM_ESHAPE instead of choosing another.
 * Every value keeps results within the stated bounds (the hand-off choices
 * change no bits at all).
 */
enum skgemm_knob {
  SKGEMM_KNOB_KIND = 0,        /* 0 one tile per workgroup, 1 persistent, 2 all
                                  ranks in one workgroup, 3 wide tiles        */
  SKGEMM_KNOB_STREAM = 1,      /* persistent kernel: shape index 0..6         */
  SKGEMM_KNOB_SHAPE = 2,       /* one-tile-per-workgroup kernel: shape 0..7   */
  SKGEMM_KNOB_FOLD = 3,        /* all-ranks kernel: largest K fold 1, 2, 4, 8 */
  SKGEMM_KNOB_CLUSTER_C = 4,   /* all-ranks kernel: bf16 pieces per lane 1, 2 */
  SKGEMM_KNOB_WG_PER_CU = 5,   /* persistent kernel: workgroups per CU        */
  SKGEMM_KNOB_PDEFER = 6,      /* persistent kernel: partials held in LDS 0/1 */
  SKGEMM_KNOB_OWNER_WAIT = 7,  /* owner wait bound, 100 MHz ticks (0: hand the
                                  tile over at once)                          */
  SKGEMM_KNOB_HANDOFF = 8      /* persistent kernel's split-K hand-off:
                                  0 arrival counter, 1 tagged mailbox         */
};
SKGEMM_API int skgemm_set_override(int knob, int value);

/* skgemm_strerror: static text for a return code. */
SKGEMM_API const char* skgemm_strerror(int code);

/* skgemm_last_hip_error: the hipError_t of the last SKGEMM_EHIP on this
 * thread (0 if none). */
SKGEMM_API int skgemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SKGEMM_H */
