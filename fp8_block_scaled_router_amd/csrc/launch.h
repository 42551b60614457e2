// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public C ABI is include/moe_fp8.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Stage timestamps of a measured forward.  While the calling thread's stamp
// is armed, the forward's kernels launch through hipExtLaunchKernel with its
// events: the stage's first dispatch records its start in `start`, and every
// dispatch records its end in `stop`, so start..stop spans the stage's
// kernels as the GPU stamps their dispatches (no marker between them).
struct StageStamp {
    hipEvent_t start;
    hipEvent_t stop;
};
StageStamp& stage_stamp();   // thread-local

template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                   Args... args) {
    StageStamp& st = stage_stamp();
    if (st.start == nullptr && st.stop == nullptr) {
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, st.start, st.stop, 0, args...);
    st.start = nullptr;
}

// Router and/or 1x128 activation quantisation, one workgroup per token.
enum { kRoute = 1, kQuant = 2 };
hipError_t launch_route_quant(const float* logits, const uint16_t* x, int M, int E, int k, int h,
                              int32_t* ids, float* tw, uint8_t* xq, float* xs, int what,
                              hipStream_t stream);

// BF16 routing logits x . wr^T (bf16 rows, fp32 accumulation) and the
// router top-k on them, 32 tokens per workgroup; logits may be null.
// h % 128 == 0, 1 <= E <= 256, 1 <= k <= min(E, 16).
hipError_t launch_router_gemm_topk(const uint16_t* x, const uint16_t* wr, int M, int h, int E, int k,
                                   float* logits, int32_t* ids, float* tw, hipStream_t stream);

// The same plus the grouping of all routes, in one launch, for batches of at
// most kGroupTailRoutes routes; arrivals is a zero word that the launch
// leaves at zero.
constexpr int kGroupTailRoutes = 256;
hipError_t launch_route_quant_group(const float* logits, const uint16_t* x, int M, int E, int k, int h,
                                    int32_t* ids, float* tw, uint8_t* xq, float* xs, int32_t* counts,
                                    int32_t* offsets, int32_t* sorted, int32_t* active,
                                    int32_t* num_active, uint32_t* arrivals, hipStream_t stream);

// Grouping of R routes by expert: per-chunk histograms, then an ordered
// scatter.  `hist` holds group_chunks(R) * E ints.
int group_chunks(int R);
hipError_t launch_group(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, int32_t* active, int32_t* num_active,
                        hipStream_t stream, int tile_m = 0, int32_t* mtile_off = nullptr);

// Weight-streaming grouped GEMMs (few tokens per expert).
struct StreamArgs {
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* active;
    const int32_t* num_active;
    int max_slots;   // upper bound on the number of distinct experts (min(E, M*k))
    int h, i, k;
};
hipError_t launch_stream_gate_up(const StreamArgs& a, const uint8_t* xq, const float* xs,
                                 const uint8_t* w13, const float* s13, float* g, hipStream_t stream);
hipError_t launch_stream_down(const StreamArgs& a, const float* g, const uint8_t* w2, const float* s2,
                              float* y, hipStream_t stream);

// The same GEMMs with MXFP4 weights (E2M1 codes two per byte along K, E8M0
// scales per 32 K elements: w13 [E][2i][h/2] + e13 [E][2i][h/32], w2
// [E][h][i/2] + e2 [E][h][i/32]).
hipError_t launch_stream_gate_up_mx(const StreamArgs& a, const uint8_t* xq, const float* xs, const uint8_t* w13,
                                    const uint8_t* e13, float* g, hipStream_t stream);
hipError_t launch_stream_down_mx(const StreamArgs& a, const float* g, const uint8_t* w2, const uint8_t* e2,
                                 float* y, hipStream_t stream);

// Tiled grouped GEMMs for many tokens per expert.
struct PrefillArgs {
    const uint8_t* xq;
    const float* xs;
    const uint8_t* w13;         // FP8 [E][2i][h], or MXFP4 codes [E][2i][h/2]
    const float* s13;           // FP8: 128x128 block scales
    const uint8_t* e13;         // MXFP4: E8M0 scales [E][2i][h/32]
    const uint8_t* w2;          // FP8 [E][h][i], or MXFP4 codes [E][h][i/2]
    const float* s2;
    const uint8_t* e2;          // MXFP4: [E][h][i/32]
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* mtile_off;   // [E + 1] first M-tile of each expert
    uint8_t* a2;                // [R][i]   requantised activations, sorted-route order
    float* a2s;                 // [R][i/128]
    uint16_t* y;                // [R][h]   bf16 partials by route id
    uint32_t* done;             // producer: gate/up tiles finished per M-tile (null otherwise)
    uint32_t* err;              // producer: the workspace's sticky error word
    int h, i, E, k;
    int weights_nt;             // FP8: nonzero copies the weight tiles with nontemporal loads
};
int prefill_tile_m();
bool prefill_supported(int M, int h, int i, int k);

// The prefill producer: routing, quantisation, grouping and both tiled
// GEMMs in one launch of one workgroup per CU (all resident), feeding the
// route reducer (launch_combine_bf16 with the error word).
struct ProducerArgs {
    PrefillArgs pa;              // the GEMMs' view of the buffers below, with done and err set
    const float* logits;
    const uint16_t* x;
    int32_t* ids;
    float* tw;
    uint8_t* xq;
    float* xs;
    int32_t* hist;               // [chunks][E] routes per expert of each routing chunk
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* num_active;
    int32_t* mtile_off;
    uint32_t* sync;              // the workspace head's synchronisation words
    int M;
    int tpw;                     // tokens per routing chunk (set by the launcher)
};
constexpr int kProdMaxGrid = 512;   // routing chunks at most (rows of hist)
bool producer_supported(int M, int h, int i, int E, int k);
hipError_t launch_prefill_producer(const ProducerArgs& p, bool mx, hipStream_t stream);
// mx: MXFP4 weights (w13 / w2 with e13 / e2), else FP8 (with s13 / s2).
hipError_t launch_prefill_gate_up(const PrefillArgs& a, bool mx, hipStream_t stream);
hipError_t launch_prefill_down(const PrefillArgs& a, bool mx, hipStream_t stream);

// Fixed-order combine of the k route partials of each token into bf16.
hipError_t launch_combine(const float* y, const float* tw, int M, int k, int h, uint16_t* out,
                          hipStream_t stream);
// Same, for bf16 partials (the prefill path).  err: when given and its
// kErrProducer bit is set (the producer gave up), every output is NaN.
hipError_t launch_combine_bf16(const uint16_t* y, const float* tw, int M, int k, int h, uint16_t* out,
                               hipStream_t stream, const uint32_t* err = nullptr);

// RMSNorm of bf16 rows fused with the 1x128 activation quantisation; y
// (bf16 [M][h], the normalised rows) may be null.  h % 128 == 0,
// h <= kFrontMaxHidden.
constexpr int kFrontMaxHidden = 8192;
hipError_t launch_rmsnorm_quant(const uint16_t* x, const float* gamma, float eps, int M, int h,
                                uint16_t* y, uint8_t* q, float* s, hipStream_t stream);

// Measurement kernels (not on the forward path): an empty kernel of `grid`
// 256-thread workgroups, and a streaming read of `bytes` (a multiple of 16)
// that leaves 4 * grid words at `sink`.
hipError_t launch_probe_empty(int grid, hipStream_t stream);
hipError_t launch_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream);

// Utilities.
hipError_t launch_quant_weight(const float* w, int64_t batch, int N, int K, uint8_t* q, float* s,
                               hipStream_t stream);
hipError_t launch_encode_e4m3(const float* in, int64_t n, uint8_t* out, hipStream_t stream);

}  // namespace moe
