/*
 * moe_fp8.h -- C ABI of the routed FP8 (E4M3, 128x128 block-scaled)
 * mixture-of-experts expert FFN for AMD Instinct MI355X (gfx950, wave64).
 *
 * The layer (stage order of the Netra Kernel README, MoE prefill pair:
 * routing, gate/up, SiLU and quantisation, down-partial, route reducer):
 *   1. router: softmax over E fp32 logits, top-k by logit (ties go to the
 *      lower expert index), weights renormalised over the k picks;
 *   2. per-token 1x128 FP8 activation quantisation (fp32 scale per 128
 *      columns, Netra compiler architecture page: FP8 activation plus
 *      fp32 activation-scale tensors);
 *   3. grouping of the M*k routes by expert (counts, offsets, routes sorted
 *      by expert then route id);
 *   4. block-scaled FP8 gate/up GEMM with FP32 results;
 *   5. SiLU(gate) * up, requantised to FP8 per 128 columns;
 *   6. block-scaled FP8 down GEMM, one partial row per route (fp32; bf16
 *      on the prefill path, inside the output tolerance);
 *   7. combine: out[t] = bf16( sum over r = 0..k-1 of w[t,r] * partial[t*k+r] ),
 *      summed in rank order with no atomic adds (Inferact amd-kernels README,
 *      atomics rule).
 * Formats (Netra Kernel README capability table; kernel-laboratory README
 * supported-targets table): E4M3 is the OCP "FN" variant (max 448, NaN at
 * 0x7F/0xFF); a block scale is amax/448 in fp32 and dequantisation is
 * code * scale; conversion to E4M3 rounds to nearest even and saturates.
 *
 * General conventions (Netra Kernel README, runtime C ABI; Netra compiler
 * architecture page, compile/init/launch flow):
 *  - Every tensor pointer is caller-owned DEVICE memory on the current HIP
 *    device, row-major and contiguous, 16-byte aligned.  Inputs are never
 *    written.  Outputs are fully overwritten.
 *  - Work is enqueued on `stream`; calls return after the enqueue.  The
 *    launch path allocates nothing and never synchronises, so a forward can
 *    be captured into a HIP graph.
 *  - Arguments are checked on the host before any HIP call; a rejected call
 *    enqueues nothing.  No C++ exception crosses the ABI.
 *  - Results are bitwise deterministic: identical inputs give identical
 *    outputs on every run.
 *  - Two forwards that share a workspace must not run concurrently (use one
 *    workspace per stream).
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = -1,      /* null pointer, negative size, misaligned pointer */
    MOE_ERR_UNSUPPORTED = -2,  /* shape outside what the kernels are built for: the caller falls back */
    MOE_ERR_WORKSPACE = -3,    /* no workspace bound / workspace too small */
    MOE_ERR_HIP = -4           /* a HIP call or kernel launch failed */
};

/* Forward paths (chosen from the sizes alone, see moe_fp8_workspace_layout):
 * one to four tokens run the whole layer in one kernel whose workgroups are
 * all resident at once, provided its grid fits 512 workgroups: every unit
 * (selected expert x 128-column block of the intermediate) is split into 8
 * or 4 parts (for h 2048, i 768, E 128, top-8 that is M <= 2); other batches
 * with few routes per expert run weight-streaming GEMMs; batches with at
 * least 8 routes per expert on average (M*k >= 8*E) and h % 256 == 0 run
 * tiled MFMA grouped GEMMs with the SiLU requantisation fused into the
 * gate/up epilogue, in five launches (routing and quantisation, grouping,
 * gate/up, down, combine).  The same tiled GEMMs also run as the prefill
 * producer and its route reducer (the Netra Kernel README's MoE prefill
 * pair, two launches: routing, quantisation, grouping and both GEMMs in one
 * kernel whose workgroups, one per CU, are all resident at once, then the
 * fixed-order combine; batches of at most 7168 - E M-tiles of 128 routes),
 * bit for bit the same result, when a caller asks for that path
 * (moe_fp8_forward_ws_path). */
#define MOE_FP8_PATH_STREAM 0
#define MOE_FP8_PATH_PREFILL 1
#define MOE_FP8_PATH_FUSED_DECODE 2
#define MOE_FP8_PATH_PRODUCER 3

/* Bits of the workspace's sticky error word (moe_fp8_workspace_status). */
#define MOE_FP8_ERR_FUSED_WAIT 1u      /* a wait of the one-kernel decode path timed out */
#define MOE_FP8_ERR_PRODUCER_WAIT 2u   /* a wait of the prefill producer timed out (its output is NaN) */

/* Shape limits of this build. */
#define MOE_FP8_MAX_EXPERTS 256
#define MOE_FP8_MAX_TOPK 16
#define MOE_FP8_MAX_HIDDEN 16384        /* h */
#define MOE_FP8_MAX_INTERMEDIATE 2048   /* i */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_fp8_status_string(int status);

/* Bytes of device workspace a forward with these sizes needs (0 for M == 0
 * or an unsupported shape). */
size_t moe_fp8_workspace_bytes(int M, int h, int i, int E, int k);

/* Workspaces.  The first 8 MiB + 32 KiB of every workspace (the "head")
 * hold synchronisation words and the exchange buffers of the one-kernel
 * small-batch path; the head must be zero before the workspace's first
 * forward and is then maintained by the forwards themselves.
 * moe_fp8_bind_workspace zeroes it; a caller-managed workspace is zeroed once
 * with moe_fp8_workspace_init (or allocated zero-filled).  The word at
 * moe_fp8_ws_layout.sync_error stays 0 unless a wait between workgroups
 * timed out (a broken device or a corrupted workspace), in which case it is
 * set and that forward's output is invalid. */

/* Reads the sticky error word of a workspace into *flags (0: every wait
 * between workgroups completed; nonzero: a wait of some earlier forward on
 * this workspace timed out and that forward's output is invalid -- it also
 * holds NaN where the late data was needed; the MOE_FP8_ERR_* bits say which
 * path), after the work already queued
 * on `stream`; with `clear` nonzero the word is then reset to 0.  `flags` is
 * host memory.  Synchronises `stream`: not for the launch path or graph
 * capture.  MOE_ERR_INVALID on a null or misaligned pointer,
 * MOE_ERR_WORKSPACE when the workspace is smaller than the head. */
int moe_fp8_workspace_status(void* workspace, size_t workspace_bytes, int clear, uint32_t* flags,
                             hipStream_t stream);

/* Bind `bytes` of device memory at `dev_ptr` (256-byte aligned) as the
 * workspace moe_fp8_forward uses on the CURRENT device, and zero its
 * synchronisation words (synchronously).  The library keeps the pointer, not
 * the memory: the caller owns it and must keep it alive while bound.
 * Passing NULL unbinds.  Not on the launch path; call it once before
 * capturing graphs.  Returns MOE_ERR_INVALID on misalignment and
 * MOE_ERR_WORKSPACE when it is smaller than the head. */
int moe_fp8_bind_workspace(void* dev_ptr, size_t bytes);

/* Bytes of the workspace head (every workspace is at least this large). */
size_t moe_fp8_workspace_head_bytes(void);

/* Zero the head of a workspace (a kernel on `stream`, so it may be
 * captured).  Needed once before the first forward on a workspace that was
 * not allocated zero-filled. */
int moe_fp8_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The whole layer with the workspace bound to the current device.
 *   x              bf16 [M, h]
 *   router_logits  fp32 [M, E]
 *   w13            e4m3 [E, 2i, h]; rows [0, i) are the gate projection,
 *                  rows [i, 2i) the up projection
 *   s13            fp32 [E, 2i/128, h/128]  (one scale per 128x128 block)
 *   w2             e4m3 [E, h, i]
 *   s2             fp32 [E, h/128, i/128]
 *   out            bf16 [M, h]
 * Requires h % 128 == 0, i % 128 == 0, 1 <= k <= min(E, 16), E <= 256.
 * M == 0 is a no-op that returns MOE_OK. */
int moe_fp8_forward(const void* x, const float* router_logits,
                    const void* w13, const float* s13,
                    const void* w2, const float* s2,
                    void* out, int M, int h, int i, int E, int k,
                    hipStream_t stream);

/* Same, with an explicit workspace of `workspace_bytes` bytes (256-byte
 * aligned device memory, at least moe_fp8_workspace_bytes(M, h, i, E, k)).
 * After the call the workspace holds the forward's intermediates at the
 * offsets moe_fp8_workspace_layout reports. */
int moe_fp8_forward_ws(const void* x, const float* router_logits,
                       const void* w13, const float* s13,
                       const void* w2, const float* s2,
                       void* out, int M, int h, int i, int E, int k,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the layer of
 * moe_fp8_forward_ws with its workspace in a fixed device array of
 * MOE_FP8_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends (zero when the module loads; the forwards
 * keep its synchronisation words consistent from then on).  The caller passes
 * only inputs and outputs, as for moe_fp8_forward.  Nothing is allocated:
 * the first call on a device looks up the array's address there.  Sizes whose
 * workspace (moe_fp8_workspace_bytes) exceeds the array -- the large-batch
 * prefill path, for one -- return MOE_ERR_WORKSPACE and enqueue nothing; the
 * caller then uses moe_fp8_forward_ws.  Every call on a device shares that
 * device's array, so calls that overlap on one device (other streams, other
 * threads) race: serialise them.  Other arguments, errors and results as
 * moe_fp8_forward_ws. */
#define MOE_FP8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_fp8_forward_noalloc(const void* x, const float* router_logits,
                            const void* w13, const float* s13,
                            const void* w2, const float* s2,
                            void* out, int M, int h, int i, int E, int k,
                            hipStream_t stream);

/* Measurement variant of moe_fp8_forward_ws: the kernels of stage j launch
 * through hipExtLaunchKernel so that events[2j] takes the GPU's timestamp of
 * the start of the stage's first dispatch and events[2j + 1] that of the end
 * of its last (hipEventElapsedTime of the pair is the stage's execution time,
 * with no marker packets between stages), for j < n =
 * moe_fp8_forward_kernel_count(...); n_events must be at least 2n, else
 * MOE_ERR_INVALID.  Stage j's kernel names are those
 * moe_fp8_forward_kernel_name reports.  The events are caller-created
 * (hipEventCreate); results are those of moe_fp8_forward_ws.  The stamps are
 * armed per calling thread. */
int moe_fp8_forward_ws_timed(const void* x, const float* router_logits,
                             const void* w13, const float* s13,
                             const void* w2, const float* s2,
                             void* out, int M, int h, int i, int E, int k,
                             void* workspace, size_t workspace_bytes,
                             hipEvent_t* events, int n_events, hipStream_t stream);

/* Measurement variant of moe_fp8_forward_ws: runs only the first n_stages
 * stages of the forward (0 <= n_stages <= moe_fp8_forward_kernel_count(...),
 * else MOE_ERR_INVALID), so that HIP-graph replays of forwards cut after
 * successive stages time each stage without events between stages.  A cut
 * forward leaves `out` and the later intermediates unwritten; with n_stages
 * equal to the stage count it is moe_fp8_forward_ws.  Same arguments,
 * ownership and errors as moe_fp8_forward_ws otherwise. */
int moe_fp8_forward_ws_prefix(const void* x, const float* router_logits,
                              const void* w13, const float* s13,
                              const void* w2, const float* s2,
                              void* out, int M, int h, int i, int E, int k,
                              void* workspace, size_t workspace_bytes,
                              int n_stages, hipStream_t stream);

/* Number of stages a forward with these sizes runs (0 for M == 0, a negative
 * status for a rejected shape) and the kernel name(s) of stage j (static
 * string, NULL when j is out of range). */
int moe_fp8_forward_kernel_count(int M, int h, int i, int E, int k);
const char* moe_fp8_forward_kernel_name(int M, int h, int i, int E, int k, int j);

/* Byte offsets of the intermediates inside a forward's workspace; a field is
 * (size_t)-1 when the path chosen for these sizes does not materialise it. */
typedef struct {
    size_t topk_ids;    /* int32 [M, k]          rank order            */
    size_t topk_w;      /* fp32  [M, k]                                 */
    size_t xq;          /* e4m3  [M, h]                                 */
    size_t xs;          /* fp32  [M, h/128]                             */
    size_t counts;      /* int32 [E]                                    */
    size_t offsets;     /* int32 [E + 1]                                */
    size_t sorted;      /* int32 [M*k]  route ids p = t*k + r           */
    size_t active;      /* int32 [E]    experts with a route, ascending */
    size_t num_active;  /* int32 [1]                                    */
    size_t gate_up;     /* fp32  [M*k, 2i]  by route id                 */
    size_t act2;        /* e4m3  [M*k, i]   in sorted-route order       */
    size_t act2_scale;  /* fp32  [M*k, i/128] in sorted-route order     */
    size_t partial;     /* [M*k, h] by route id: fp32 on the streaming path, bf16 on the prefill path */
    size_t sync_error;  /* uint32 error word (0 = no wait timed out)    */
    size_t total;       /* bytes                                        */
    int    path;        /* MOE_FP8_PATH_*                               */
} moe_fp8_ws_layout;

/* Fills *layout for these sizes.  Returns MOE_ERR_UNSUPPORTED / INVALID as
 * moe_fp8_forward would. */
int moe_fp8_workspace_layout(int M, int h, int i, int E, int k, moe_fp8_ws_layout* layout);

/* Measurement and testing: the forward on a given path (MOE_FP8_PATH_*)
 * instead of the one the library picks, with a workspace of at least
 * moe_fp8_workspace_bytes_path bytes (laid out as
 * moe_fp8_workspace_layout_path reports).  MOE_ERR_UNSUPPORTED (size 0) when
 * the path cannot take the batch: the one-kernel path beyond its grid, the
 * tiled paths for h % 256 != 0, the producer beyond its M-tile count.  The
 * results are bitwise those of the same arithmetic on any path that shares
 * it (the two tiled paths give the same bits). */
size_t moe_fp8_workspace_bytes_path(int M, int h, int i, int E, int k, int path);
int moe_fp8_workspace_layout_path(int M, int h, int i, int E, int k, int path, moe_fp8_ws_layout* layout);
int moe_fp8_forward_ws_path(const void* x, const float* router_logits,
                            const void* w13, const float* s13,
                            const void* w2, const float* s2,
                            void* out, int M, int h, int i, int E, int k,
                            void* workspace, size_t workspace_bytes, int path, hipStream_t stream);

/* Step 1 alone (the same kernel the forward runs): the routing stage that
 * opens the Netra Kernel README's MoE prefill pair and the M=1 MoE objects of
 * the Netra compiler architecture page (scope paragraph).
 *   logits fp32 [M, E] -> topk_ids int32 [M, k] (rank order: descending
 *   logit, ties to the lower expert index), topk_w fp32 [M, k] (softmax
 *   probabilities of the picks renormalised to sum to 1). */
int router_topk(const float* logits, int M, int E, int k,
                int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* BF16 routing, the step before step 1 (Netra Kernel README capability
 * table: BF16 routing among the gfx950 operation families), fused with the
 * top-k of router_topk in one launch:
 *   x bf16 [M, h] (hidden rows), wr bf16 [E, h] (router weight, one row per
 *   expert) -> logits fp32 [M, E] = x . wr^T (optional: null skips the
 *   store), topk_ids int32 [M, k] and topk_w fp32 [M, k] exactly as
 *   router_topk computes them from those logits.
 * The products are exact; the sums are fp32 matrix-core accumulations, so a
 * logit may differ from the correctly rounded sum by a small multiple of
 * 2^-24 * sum_j |x_j wr_j|, and two experts whose logits lie that close may
 * swap ranks.  Deterministic: the same inputs give the same bits, and a
 * token's logits do not depend on M or on whether `logits` is null.  With
 * `logits` non-null and M <= 4064 the call is two launches (the logits spread
 * over workgroups by expert, then router_topk's kernel on them); otherwise
 * one launch computes the logits and the top-k together.
 * All buffers are caller-owned device memory; x and wr 16-byte aligned.
 * h % 128 == 0 and h <= MOE_FP8_MAX_HIDDEN, E <= MOE_FP8_MAX_EXPERTS,
 * 1 <= k <= min(E, MOE_FP8_MAX_TOPK) (else MOE_ERR_UNSUPPORTED); a null or
 * misaligned pointer or a negative size gives MOE_ERR_INVALID; M == 0 is a
 * no-op.  Enqueued on `stream`. */
int moe_fp8_router_gemm_topk(const void* x, const void* wr, int M, int h, int E, int k,
                             float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* The layer with MXFP4 expert weights (Inferact amd-kernels README, naming
 * section: moe/mxfp4_h6144_i768_e128_top4; Netra Kernel README, targets
 * table: MXFP4 checkpoints).  Weights are OCP MX FP4: E2M1 codes packed two
 * per byte along K (element 2j in the low nibble of byte j) with one E8M0
 * scale (2^(c - 127)) per 32 consecutive K elements:
 *   w13 [E, 2i, h/2] codes + e13 [E, 2i, h/32] scales (rows [0,i) gate),
 *   w2  [E, h, i/2]  codes + e2  [E, h, i/32]  scales.
 * Routing, the 1x128 E4M3 activation quantisation, the SiLU-mul
 * requantisation and the rank-order combine are those of moe_fp8_forward;
 * the GEMMs run on the block-scaled FP4 x FP8 matrix cores and accumulate in
 * fp32 (the result differs from the float64 dequantised reference by the
 * matrix cores' block-sum rounding).  Batches with M*k >= 12*E take the
 * tiled kernels of the FP8 prefill path (bf16 partials, as there; the
 * producer and its reducer on request) when h % 256 == 0; the rest take the
 * weight-streaming kernels (fp32 partials).
 * The workspace (>= moe_mxfp4_workspace_bytes,
 * 256-byte aligned) follows the rules of moe_fp8_forward_ws: its head must
 * be zero before the first forward (moe_fp8_workspace_init).  x, logits, out,
 * w13 and w2 16-byte aligned, e13 and e2 4-byte aligned, else
 * MOE_ERR_INVALID; shapes as moe_fp8_forward_ws.  Enqueued on `stream`. */
size_t moe_mxfp4_workspace_bytes(int M, int h, int i, int E, int k);
/* The workspace layout of an MXFP4 forward with these sizes, as
 * moe_fp8_workspace_layout (path is MOE_FP8_PATH_STREAM, _PREFILL or
 * _PRODUCER). */
int moe_mxfp4_workspace_layout(int M, int h, int i, int E, int k, moe_fp8_ws_layout* layout);
/* Measurement: the same forward with the stage stamps of
 * moe_fp8_forward_ws_timed (events[2j], events[2j + 1]: start of stage j's
 * first dispatch, end of its last; n_events >= 2 * the stage count, else
 * MOE_ERR_INVALID). */
/* The MXFP4 forward on a given path (MOE_FP8_PATH_STREAM, _PREFILL or
 * _PRODUCER), as moe_fp8_forward_ws_path. */
size_t moe_mxfp4_workspace_bytes_path(int M, int h, int i, int E, int k, int path);
int moe_mxfp4_forward_ws_path(const void* x, const float* router_logits,
                              const void* w13, const void* e13, const void* w2, const void* e2,
                              void* out, int M, int h, int i, int E, int k,
                              void* workspace, size_t workspace_bytes, int path, hipStream_t stream);
int moe_mxfp4_forward_ws_timed(const void* x, const float* router_logits,
                               const void* w13, const void* e13, const void* w2, const void* e2,
                               void* out, int M, int h, int i, int E, int k,
                               void* workspace, size_t workspace_bytes,
                               hipEvent_t* events, int n_events, hipStream_t stream);
/* Stage count and kernel name(s) of stage j of an MXFP4 forward with these
 * sizes, as moe_fp8_forward_kernel_count / _name. */
int moe_mxfp4_forward_kernel_count(int M, int h, int i, int E, int k);
const char* moe_mxfp4_forward_kernel_name(int M, int h, int i, int E, int k, int j);
int moe_mxfp4_forward_ws(const void* x, const float* router_logits,
                         const void* w13, const void* e13, const void* w2, const void* e2,
                         void* out, int M, int h, int i, int E, int k,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Measurement: the same forward cut after its first n_stages launches (the
 * stages are route+quant(+group), [group], gate/up, down, combine; graph
 * replays of cut forwards give per-stage durations).  n_stages < 0 gives
 * MOE_ERR_INVALID. */
int moe_mxfp4_forward_ws_prefix(const void* x, const float* router_logits,
                                const void* w13, const void* e13, const void* w2, const void* e2,
                                void* out, int M, int h, int i, int E, int k,
                                void* workspace, size_t workspace_bytes, int n_stages,
                                hipStream_t stream);

/* Step 2 alone (the FP8 activation and fp32 activation-scale tensors of the
 * Netra compiler architecture page, compatibility-engine paragraph):
 * rows of bf16 [M, K] -> q e4m3 [M, K], s fp32 [M, K/128];
 * s = amax/448 of each 1x128 group, q = E4M3(x / s), all-zero groups give
 * s = 0 and zero codes.  K % 128 == 0. */
int moe_fp8_act_quant(const void* x, int M, int K, uint8_t* q, float* s,
                      hipStream_t stream);

/* The step before step 2 (the gfx950 "normalization and quantization
 * fusions" family of the Netra Kernel README directory map): RMSNorm of bf16
 * rows fused with the 1x128 quantisation, one pass over x.
 *   x     bf16 [M, h] (device, 16-byte aligned, read only)
 *   gamma fp32 [h], the norm weight (pass 1 + w for a zero-centred weight w)
 *   eps   >= 0, finite
 *   y     bf16 [M, h] normalised rows, or NULL when not wanted
 *   q, s  e4m3 [M, h] and fp32 [M, h/128], exactly what moe_fp8_act_quant
 *         gives for y
 * Per row: ss = sum of x^2 (exact squares, float64 sum), r = fp32(1 /
 * sqrt(ss/h + eps)) computed in float64 and rounded once, y = bf16_rne(
 * fp32(fp32(x * r) * gamma)).  All buffers are caller-owned device memory.
 * h % 128 == 0 and h <= 8192 (else MOE_ERR_UNSUPPORTED); a null or
 * misaligned pointer, M < 0 or a bad eps gives MOE_ERR_INVALID; M == 0 is a
 * no-op.  Enqueued on `stream`. */
int moe_fp8_rmsnorm_act_quant(const void* x, const float* gamma, float eps, int M, int h,
                              void* y, uint8_t* q, float* s, hipStream_t stream);

/* Step 3 alone (the routing metadata the Netra Kernel README's MoE prefill
 * producer emits for its route reducer; the activation packing of the kernel
 * laboratory README's MoE entry): topk_ids int32 [M*k] with values in [0, E) ->
 *   counts int32 [E], offsets int32 [E + 1] (exclusive scan of counts),
 *   sorted_route_ids int32 [M*k] (route ids grouped by expert ascending and
 *   ascending inside each expert).
 * Uses `workspace` (device, >= moe_fp8_group_workspace_bytes(M, E, k)). */
size_t moe_fp8_group_workspace_bytes(int M, int E, int k);
int moe_fp8_group(const int32_t* topk_ids, int M, int E, int k,
                  int32_t* counts, int32_t* offsets, int32_t* sorted_route_ids,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Weight preparation (not on the forward path): fp32 [batch, N, K] ->
 * codes e4m3 [batch, N, K] and scales fp32 [batch, N/128, K/128], one scale
 * amax/448 per 128x128 block.  N % 128 == 0, K % 128 == 0. */
int moe_fp8_quantize_weight_block128(const float* w, int64_t batch, int N, int K,
                                     uint8_t* q, float* s, hipStream_t stream);

/* Measurement helpers (not on the forward path; they frame the layer's
 * timings, Netra Kernel README kernel laboratory, rules: every number says
 * how it was taken).  moe_fp8_probe_empty enqueues an empty kernel of `grid`
 * 256-thread workgroups (the cost of a launch by itself in a graph).
 * moe_fp8_probe_read enqueues one kernel of `grid` workgroups that streams
 * `bytes` (a multiple of 16) from device memory `src` (16-byte aligned) and
 * writes 4 * grid words of xor folds to device memory `sink` (the HBM read
 * rate one launch reaches on that many bytes).  MOE_ERR_INVALID on a null or
 * misaligned pointer, a ragged size or grid outside [1, 2^20]. */
int moe_fp8_probe_empty(int grid, hipStream_t stream);
int moe_fp8_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream);

/* The device E4M3 encoder every kernel uses, applied elementwise:
 * out[j] = E4M3(in[j]) (nearest, ties to even, saturating to +-448). */
int moe_fp8_encode_e4m3(const float* in, int64_t n, uint8_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP8_H */
