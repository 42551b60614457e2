// moe_fp8.hip -- the C ABI (include/moe_fp8.h): argument checks, workspace
// layout, per-device workspace binding and the enqueue of the layer's
// kernels on the caller's stream.
//
// Interface style follows the Netra Kernel README (runtime C ABI: bind
// persistent buffers, launch on a caller-provided stream) and the Netra
// compiler architecture page (compile/init/launch flow: the launch path does
// a numeric guard and launches, with no allocation, lookup or parsing;
// unsupported contracts return a fallback status).
#include <mutex>

#include "../../include/moe_fp8.h"
#include "fused_decode.h"
#include "launch.h"

namespace moe {
StageStamp& stage_stamp() {
    static thread_local StageStamp s{nullptr, nullptr};
    return s;
}
}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Binding {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_bind_mu;
Binding g_bind[kMaxDevices];

// Workspace of moe_fp8_forward_noalloc: one fixed array per device, zero at
// module load.  Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address
// looked up once per device below.
constexpr size_t kScratchBytes = MOE_FP8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Shape checks shared by every entry point of the layer.
int check_shape(int M, int h, int i, int E, int k) {
    if (M < 0 || h <= 0 || i <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID;
    if (h % 128 != 0 || i % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (h > MOE_FP8_MAX_HIDDEN || i > MOE_FP8_MAX_INTERMEDIATE) return MOE_ERR_UNSUPPORTED;
    if (E > MOE_FP8_MAX_EXPERTS || k > MOE_FP8_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)M * k > (int64_t)1 << 28) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

struct Layout {
    moe_fp8_ws_layout pub;
    size_t hist;        // grouping scratch: group_chunks(R) * E ints
    size_t mtile_off;   // prefill path: [E + 1] ints
};

// The one-kernel decode path takes every batch it supports: its grid (one
// workgroup per eighth or quarter of an (expert, 128-column intermediate
// block) unit, for every expert the batch could select) must be resident at
// once, which limits it to one or two tokens at the layer shapes.  Above it,
// the tiled kernels take over from the weight-streaming ones at 8 routes per
// expert on average: the streaming kernels read each weight tile once per 16
// routes of its expert, and at h 2048 / 6144, i 768, E 128 the two cost the
// same between 4 and 8 routes per expert (measured).
constexpr int kTiledRoutesPerExpert = 8;
// MXFP4 weights halve the bytes the streaming kernels read per pass, which
// moves the crossover to between 8 and 16 routes per expert (measured at the
// same shapes).
constexpr int kTiledRoutesPerExpertMx = 12;

// Whether a batch of these sizes can take the path (the MXFP4 layer has no
// one-kernel path).
bool path_ok(int path, int M, int h, int i, int E, int k, bool mx) {
    switch (path) {
        case MOE_FP8_PATH_STREAM: return true;
        case MOE_FP8_PATH_PREFILL: return moe::prefill_supported(M, h, i, k);
        case MOE_FP8_PATH_PRODUCER: return moe::producer_supported(M, h, i, E, k);
        case MOE_FP8_PATH_FUSED_DECODE: return !mx && moe::fused_supported(M, h, i, E, k);
        default: return false;
    }
}

// The tiled kernels run as five launches by default: the producer and its
// reducer (two launches, the same bits) measured 5-7% slower from 768 to
// 8192 tokens at h 2048, i 768, E 128, top-8 (its in-kernel grid barriers
// and the device-scope stores of everything handed across them cost more
// than the launch boundaries they replace), and 3% faster at 256 tokens; it
// runs when asked for (moe_fp8_forward_ws_path).
int tiled_path(int M, int h, int i, int E, int k) {
    (void)E;
    if (moe::prefill_supported(M, h, i, k)) return MOE_FP8_PATH_PREFILL;
    return MOE_FP8_PATH_STREAM;
}

int choose_path(int M, int h, int i, int E, int k) {
    if (moe::fused_supported(M, h, i, E, k)) return MOE_FP8_PATH_FUSED_DECODE;
    if ((int64_t)M * k >= (int64_t)kTiledRoutesPerExpert * E) return tiled_path(M, h, i, E, k);
    return MOE_FP8_PATH_STREAM;
}

int choose_path_mx(int M, int h, int i, int E, int k) {
    if ((int64_t)M * k >= (int64_t)kTiledRoutesPerExpertMx * E) return tiled_path(M, h, i, E, k);
    return MOE_FP8_PATH_STREAM;
}

// path < 0: the path the library picks for these sizes.
void make_layout(int M, int h, int i, int E, int k, Layout* L, bool mx = false, int path = -1) {
    const size_t R = (size_t)M * k;
    size_t cur = moe::kWorkspaceHead;   // synchronisation words and exchange region first
    auto take = [&](size_t bytes) {
        const size_t o = cur;
        cur = align_up(cur + bytes);
        return o;
    };
    moe_fp8_ws_layout& p = L->pub;
    p.sync_error = moe::kSyncErr;
    p.topk_ids = take(R * 4);
    p.topk_w = take(R * 4);
    p.xq = take((size_t)M * h);
    p.xs = take((size_t)M * (h / 128) * 4);
    p.counts = take((size_t)E * 4);
    p.offsets = take((size_t)(E + 1) * 4);
    p.sorted = take(R * 4);
    p.active = take((size_t)E * 4);
    p.num_active = take(4);
    p.path = path >= 0 ? path : mx ? choose_path_mx(M, h, i, E, k) : choose_path(M, h, i, E, k);
    // grouping scratch: the chunk counts (the producer's chunks are at most
    // one per workgroup of its grid)
    const size_t chunks = (size_t)moe::group_chunks((int)R);
    L->hist = take((p.path == MOE_FP8_PATH_PRODUCER ? std::max(chunks, (size_t)moe::kProdMaxGrid) : chunks) * E * 4);
    L->mtile_off = take((size_t)(E + 1) * 4);
    p.gate_up = (size_t)-1;
    p.act2 = (size_t)-1;
    p.act2_scale = (size_t)-1;
    p.partial = (size_t)-1;
    if (p.path == MOE_FP8_PATH_STREAM) {
        p.gate_up = take(R * 2 * i * 4);
        p.partial = take(R * h * 4);
    } else if (p.path == MOE_FP8_PATH_PREFILL || p.path == MOE_FP8_PATH_PRODUCER) {
        p.act2 = take(R * i);
        p.act2_scale = take(R * (i / 128) * 4);
        p.partial = take(R * h * 2);   // bf16 partials
    }   // the fused path exchanges its intermediates as tagged words in the head
    p.total = cur;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Kernels of one forward, in launch order, per path.
const char* const kStreamStages[] = {"route_quant_kernel", "group_hist+group_scatter",
                                     "stream_gate_up_kernel", "stream_down_kernel",
                                     "combine_kernel"};
const char* const kStreamSmallStages[] = {"route_quant_group_kernel", "stream_gate_up_kernel",
                                          "stream_down_kernel", "combine_kernel"};
const char* const kFusedStages[] = {"fused_decode_kernel"};
const char* const kPrefillStages[] = {"route_quant_kernel", "group_hist+group_scatter",
                                      "prefill_gate_up_kernel", "prefill_down_kernel",
                                      "combine_bf16_kernel"};
const char* const kStreamMxStages[] = {"route_quant_kernel", "group_hist+group_scatter",
                                       "stream_gate_up_mx_kernel", "stream_down_mx_kernel",
                                       "combine_kernel"};
const char* const kStreamSmallMxStages[] = {"route_quant_group_kernel", "stream_gate_up_mx_kernel",
                                            "stream_down_mx_kernel", "combine_kernel"};
const char* const kPrefillMxStages[] = {"route_quant_kernel", "group_hist+group_scatter",
                                        "prefill_gate_up_mx_kernel", "prefill_down_mx_kernel",
                                        "combine_bf16_kernel"};
const char* const kProducerStages[] = {"prefill_producer_kernel", "combine_bf16_kernel"};
const char* const kProducerMxStages[] = {"prefill_producer_mx_kernel", "combine_bf16_kernel"};

// The streaming path routes, quantises and groups in one launch when the
// batch has few enough routes.
bool small_group(int M, int k) { return (int64_t)M * k <= moe::kGroupTailRoutes; }

int stage_count(int path, int M, int k) {
    if (path == MOE_FP8_PATH_FUSED_DECODE) return 1;
    if (path == MOE_FP8_PATH_PRODUCER) return 2;
    if (path == MOE_FP8_PATH_STREAM && small_group(M, k)) return 4;
    return 5;
}
const char* stage_name(int path, int M, int k, int j) {
    if (path == MOE_FP8_PATH_FUSED_DECODE) return kFusedStages[j];
    if (path == MOE_FP8_PATH_PREFILL) return kPrefillStages[j];
    if (path == MOE_FP8_PATH_PRODUCER) return kProducerStages[j];
    if (small_group(M, k)) return kStreamSmallStages[j];
    return kStreamStages[j];
}
const char* stage_name_mx(int path, int M, int k, int j) {
    if (path == MOE_FP8_PATH_PREFILL) return kPrefillMxStages[j];
    if (path == MOE_FP8_PATH_PRODUCER) return kProducerMxStages[j];
    if (small_group(M, k)) return kStreamSmallMxStages[j];
    return kStreamMxStages[j];
}

// Stage bookkeeping of one forward: optional timing events per stage
// (events[2j] and events[2j + 1] take the GPU's stamps of the start of stage
// j's first dispatch and the end of its last; armed on this thread while the
// stage launches), and an optional cut after `limit` stages.
struct EventHook {
    hipEvent_t* ev;
    int n;
    int next = 0;   // stage whose events come next
    hipStream_t s;
    int limit = 1 << 30;
    int stage = 0;
    void arm() {
        if (ev && 2 * next + 1 < n) moe::stage_stamp() = moe::StageStamp{ev[2 * next], ev[2 * next + 1]};
        ++next;
    }
    static void disarm() { moe::stage_stamp() = moe::StageStamp{nullptr, nullptr}; }
    bool cut() { return stage++ >= limit; }
};

// One stage of a forward: the cut of a measurement forward, the stage's
// timing stamps, the launch.
#define MOE_STEP(call)                 \
    do {                               \
        if (hook.cut()) return MOE_OK; \
        hook.arm();                    \
        rc = hip_status(call);         \
        EventHook::disarm();           \
        if (rc != MOE_OK) return rc;   \
    } while (0)

// The tiled paths, for FP8 (s13, s2) or MXFP4 (e13, e2) weights: routing
// with quantisation, grouping, the gate/up and down GEMMs and the bf16
// reducer in five launches, or the producer and the reducer in two.
int tiled_forward(const Layout& L, void* workspace, const void* x, const float* router_logits, const void* w13,
                  const float* s13, const void* e13, const void* w2, const float* s2, const void* e2, void* out,
                  int M, int h, int i, int E, int k, EventHook& hook, hipStream_t stream) {
    int rc = MOE_OK;
    const moe_fp8_ws_layout& p = L.pub;
    const bool mx = e13 != nullptr;
    int32_t* ids = at<int32_t>(workspace, p.topk_ids);
    float* tw = at<float>(workspace, p.topk_w);
    uint8_t* xq = at<uint8_t>(workspace, p.xq);
    float* xs = at<float>(workspace, p.xs);
    int32_t* counts = at<int32_t>(workspace, p.counts);
    int32_t* offsets = at<int32_t>(workspace, p.offsets);
    int32_t* sorted = at<int32_t>(workspace, p.sorted);
    int32_t* active = at<int32_t>(workspace, p.active);
    int32_t* num_active = at<int32_t>(workspace, p.num_active);
    int32_t* hist = at<int32_t>(workspace, L.hist);
    int32_t* mtile_off = at<int32_t>(workspace, L.mtile_off);
    uint32_t* sync = at<uint32_t>(workspace, 0);
    moe::PrefillArgs pa;
    pa.xq = xq;
    pa.xs = xs;
    pa.w13 = static_cast<const uint8_t*>(w13);
    pa.s13 = s13;
    pa.e13 = static_cast<const uint8_t*>(e13);
    pa.w2 = static_cast<const uint8_t*>(w2);
    pa.s2 = s2;
    pa.e2 = static_cast<const uint8_t*>(e2);
    pa.offsets = offsets;
    pa.sorted = sorted;
    pa.mtile_off = mtile_off;
    pa.a2 = at<uint8_t>(workspace, p.act2);
    pa.a2s = at<float>(workspace, p.act2_scale);
    pa.y = at<uint16_t>(workspace, p.partial);
    pa.done = nullptr;
    pa.err = nullptr;
    pa.h = h;
    pa.i = i;
    pa.E = E;
    pa.k = k;
    // With at most 64 routes per expert on average most experts fill one
    // 128-route tile, so each FP8 weight tile is copied once per forward and
    // need not stay in the caches; with more, the route tiles of an expert
    // share its weight tiles through the L2.  (The 64-byte MXFP4 rows keep
    // ordinary copies: the two K blocks of a 128-byte line go out in
    // different stages.)
    pa.weights_nt = !mx && (int64_t)M * k <= (int64_t)64 * E;
    uint16_t* o = static_cast<uint16_t*>(out);
    if (p.path == MOE_FP8_PATH_PRODUCER) {
        pa.done = sync + moe::kSyncProdDone / 4;
        pa.err = sync + moe::kSyncErr / 4;
        moe::ProducerArgs pp;
        pp.pa = pa;
        pp.logits = router_logits;
        pp.x = static_cast<const uint16_t*>(x);
        pp.ids = ids;
        pp.tw = tw;
        pp.xq = xq;
        pp.xs = xs;
        pp.hist = hist;
        pp.counts = counts;
        pp.offsets = offsets;
        pp.sorted = sorted;
        pp.active = active;
        pp.num_active = num_active;
        pp.mtile_off = mtile_off;
        pp.sync = sync;
        pp.M = M;
        pp.tpw = 0;
        MOE_STEP(moe::launch_prefill_producer(pp, mx, stream));
        MOE_STEP(moe::launch_combine_bf16(pa.y, tw, M, k, h, o, stream, pa.err));
        return MOE_OK;
    }
    MOE_STEP(moe::launch_route_quant(router_logits, static_cast<const uint16_t*>(x), M, E, k, h, ids, tw, xq, xs,
                                     moe::kRoute | moe::kQuant, stream));
    MOE_STEP(moe::launch_group(ids, M * k, E, hist, counts, offsets, sorted, active, num_active, stream,
                               moe::prefill_tile_m(), mtile_off));
    MOE_STEP(moe::launch_prefill_gate_up(pa, mx, stream));
    MOE_STEP(moe::launch_prefill_down(pa, mx, stream));
    MOE_STEP(moe::launch_combine_bf16(pa.y, tw, M, k, h, o, stream));
    return MOE_OK;
}

int run_forward(const void* x, const float* router_logits, const void* w13, const float* s13,
                const void* w2, const float* s2, void* out, int M, int h, int i, int E, int k,
                void* workspace, size_t workspace_bytes, hipEvent_t* events, int n_events,
                hipStream_t stream, int n_stages = 1 << 30, int path = -1) {
    int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return MOE_OK;
    if (!x || !router_logits || !w13 || !s13 || !w2 || !s2 || !out) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(router_logits) || !aligned16(w13) || !aligned16(s13) ||
        !aligned16(w2) || !aligned16(s2) || !aligned16(out))
        return MOE_ERR_INVALID;
    if (path >= 0 && !path_ok(path, M, h, i, E, k, false)) return MOE_ERR_UNSUPPORTED;
    Layout L;
    make_layout(M, h, i, E, k, &L, false, path);
    if (!workspace || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < L.pub.total)
        return MOE_ERR_WORKSPACE;

    const moe_fp8_ws_layout& p = L.pub;
    const int R = M * k;
    int32_t* ids = at<int32_t>(workspace, p.topk_ids);
    float* tw = at<float>(workspace, p.topk_w);
    uint8_t* xq = at<uint8_t>(workspace, p.xq);
    float* xs = at<float>(workspace, p.xs);
    int32_t* counts = at<int32_t>(workspace, p.counts);
    int32_t* offsets = at<int32_t>(workspace, p.offsets);
    int32_t* sorted = at<int32_t>(workspace, p.sorted);
    int32_t* active = at<int32_t>(workspace, p.active);
    int32_t* num_active = at<int32_t>(workspace, p.num_active);
    int32_t* hist = at<int32_t>(workspace, L.hist);
    float* g = p.path == MOE_FP8_PATH_STREAM ? at<float>(workspace, p.gate_up) : nullptr;
    float* y = p.path != MOE_FP8_PATH_FUSED_DECODE ? at<float>(workspace, p.partial) : nullptr;
    EventHook hook{events, n_events, 0, stream, n_stages};
    uint32_t* sync = at<uint32_t>(workspace, 0);


    if (p.path == MOE_FP8_PATH_FUSED_DECODE) {
        moe::FusedArgs fa;
        fa.x = static_cast<const uint16_t*>(x);
        fa.logits = router_logits;
        fa.w13 = static_cast<const uint8_t*>(w13);
        fa.s13 = s13;
        fa.w2 = static_cast<const uint8_t*>(w2);
        fa.s2 = s2;
        fa.out = static_cast<uint16_t*>(out);
        fa.M = M;
        fa.h = h;
        fa.i = i;
        fa.E = E;
        fa.k = k;
        fa.ids = ids;
        fa.tw = tw;
        fa.xq = xq;
        fa.xs = xs;
        fa.counts = counts;
        fa.offsets = offsets;
        fa.sorted = sorted;
        fa.active = active;
        fa.num_active = num_active;
        fa.v_ll = at<uint64_t>(workspace, moe::kLLOffset);
        fa.t_ll = fa.v_ll + moe::fused_v_words(M, i, k);
        fa.sync = sync;
        MOE_STEP(moe::launch_fused_decode(fa, stream));
        return MOE_OK;
    }
    if (p.path == MOE_FP8_PATH_PREFILL || p.path == MOE_FP8_PATH_PRODUCER)
        return tiled_forward(L, workspace, x, router_logits, w13, s13, nullptr, w2, s2, nullptr, out, M, h, i, E, k,
                             hook, stream);
    if (small_group(M, k)) {
        MOE_STEP(moe::launch_route_quant_group(router_logits, static_cast<const uint16_t*>(x), M, E, k, h,
                                               ids, tw, xq, xs, counts, offsets, sorted, active,
                                               num_active, sync + moe::kSyncArrive / 4, stream));
    } else {
        MOE_STEP(moe::launch_route_quant(router_logits, static_cast<const uint16_t*>(x), M, E, k, h,
                                         ids, tw, xq, xs, moe::kRoute | moe::kQuant, stream));
    }
    if (!small_group(M, k))
        MOE_STEP(moe::launch_group(ids, R, E, hist, counts, offsets, sorted, active, num_active,
                                   stream));
    moe::StreamArgs sa;
    sa.offsets = offsets;
    sa.sorted = sorted;
    sa.active = active;
    sa.num_active = num_active;
    sa.max_slots = E < R ? E : R;
    sa.h = h;
    sa.i = i;
    sa.k = k;
    MOE_STEP(moe::launch_stream_gate_up(sa, xq, xs, static_cast<const uint8_t*>(w13), s13, g,
                                        stream));
    MOE_STEP(moe::launch_stream_down(sa, g, static_cast<const uint8_t*>(w2), s2, y, stream));
    MOE_STEP(moe::launch_combine(y, tw, M, k, h, static_cast<uint16_t*>(out), stream));
    return MOE_OK;
}

// The MXFP4-weight layer: routing, quantisation and grouping as in the FP8
// layer, then either the MXFP4 streaming GEMMs and the fp32 combine, or (large
// batches) the tiled MXFP4 GEMMs and the bf16 combine.
int run_forward_mx(const void* x, const float* router_logits, const void* w13, const void* e13, const void* w2,
                   const void* e2, void* out, int M, int h, int i, int E, int k, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, int n_stages = 1 << 30,
                   hipEvent_t* events = nullptr, int n_events = 0, int path = -1) {
    int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return MOE_OK;
    if (!x || !router_logits || !w13 || !e13 || !w2 || !e2 || !out) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(router_logits) || !aligned16(w13) || !aligned16(w2) || !aligned16(out) ||
        ((uintptr_t)e13 & 3u) != 0 || ((uintptr_t)e2 & 3u) != 0)
        return MOE_ERR_INVALID;
    if (path >= 0 && !path_ok(path, M, h, i, E, k, true)) return MOE_ERR_UNSUPPORTED;
    Layout L;
    make_layout(M, h, i, E, k, &L, true, path);
    if (!workspace || ((uintptr_t)workspace % kAlign) != 0 || workspace_bytes < L.pub.total)
        return MOE_ERR_WORKSPACE;
    const moe_fp8_ws_layout& p = L.pub;
    const int R = M * k;
    int32_t* ids = at<int32_t>(workspace, p.topk_ids);
    float* tw = at<float>(workspace, p.topk_w);
    uint8_t* xq = at<uint8_t>(workspace, p.xq);
    float* xs = at<float>(workspace, p.xs);
    int32_t* counts = at<int32_t>(workspace, p.counts);
    int32_t* offsets = at<int32_t>(workspace, p.offsets);
    int32_t* sorted = at<int32_t>(workspace, p.sorted);
    int32_t* active = at<int32_t>(workspace, p.active);
    int32_t* num_active = at<int32_t>(workspace, p.num_active);
    int32_t* hist = at<int32_t>(workspace, L.hist);
    uint32_t* sync = at<uint32_t>(workspace, 0);
    EventHook hook{events, n_events, 0, stream, n_stages};
    if (p.path == MOE_FP8_PATH_PREFILL || p.path == MOE_FP8_PATH_PRODUCER)
        return tiled_forward(L, workspace, x, router_logits, w13, nullptr, e13, w2, nullptr, e2, out, M, h, i, E, k,
                             hook, stream);
    float* g = at<float>(workspace, p.gate_up);
    float* y = at<float>(workspace, p.partial);
    if (small_group(M, k)) {
        MOE_STEP(moe::launch_route_quant_group(router_logits, static_cast<const uint16_t*>(x), M, E, k, h, ids, tw,
                                               xq, xs, counts, offsets, sorted, active, num_active,
                                               sync + moe::kSyncArrive / 4, stream));
    } else {
        MOE_STEP(moe::launch_route_quant(router_logits, static_cast<const uint16_t*>(x), M, E, k, h, ids, tw, xq,
                                         xs, moe::kRoute | moe::kQuant, stream));
        MOE_STEP(moe::launch_group(ids, R, E, hist, counts, offsets, sorted, active, num_active, stream));
    }
    moe::StreamArgs sa;
    sa.offsets = offsets;
    sa.sorted = sorted;
    sa.active = active;
    sa.num_active = num_active;
    sa.max_slots = E < R ? E : R;
    sa.h = h;
    sa.i = i;
    sa.k = k;
    MOE_STEP(moe::launch_stream_gate_up_mx(sa, xq, xs, static_cast<const uint8_t*>(w13),
                                           static_cast<const uint8_t*>(e13), g, stream));
    MOE_STEP(moe::launch_stream_down_mx(sa, g, static_cast<const uint8_t*>(w2), static_cast<const uint8_t*>(e2),
                                        y, stream));
    MOE_STEP(moe::launch_combine(y, tw, M, k, h, static_cast<uint16_t*>(out), stream));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_mxfp4_workspace_layout(int M, int h, int i, int E, int k, moe_fp8_ws_layout* layout) {
    if (!layout) return MOE_ERR_INVALID;
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    Layout L;
    make_layout(M, h, i, E, k, &L, true);
    *layout = L.pub;
    return MOE_OK;
}

size_t moe_mxfp4_workspace_bytes_path(int M, int h, int i, int E, int k, int path) {
    if (M == 0 || check_shape(M, h, i, E, k) != MOE_OK || !path_ok(path, M, h, i, E, k, true)) return 0;
    Layout L;
    make_layout(M, h, i, E, k, &L, true, path);
    return L.pub.total;
}

int moe_mxfp4_forward_ws_path(const void* x, const float* router_logits, const void* w13, const void* e13,
                              const void* w2, const void* e2, void* out, int M, int h, int i, int E, int k,
                              void* workspace, size_t workspace_bytes, int path, hipStream_t stream) {
    if (path < 0) return MOE_ERR_INVALID;
    return run_forward_mx(x, router_logits, w13, e13, w2, e2, out, M, h, i, E, k, workspace, workspace_bytes,
                          stream, 1 << 30, nullptr, 0, path);
}

int moe_mxfp4_forward_kernel_count(int M, int h, int i, int E, int k) {
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return 0;
    return stage_count(choose_path_mx(M, h, i, E, k), M, k);
}

const char* moe_mxfp4_forward_kernel_name(int M, int h, int i, int E, int k, int j) {
    const int n = moe_mxfp4_forward_kernel_count(M, h, i, E, k);
    if (n <= 0 || j < 0 || j >= n) return nullptr;
    return stage_name_mx(choose_path_mx(M, h, i, E, k), M, k, j);
}

size_t moe_mxfp4_workspace_bytes(int M, int h, int i, int E, int k) {
    if (M == 0 || check_shape(M, h, i, E, k) != MOE_OK) return 0;
    Layout L;
    make_layout(M, h, i, E, k, &L, true);
    return L.pub.total;
}

int moe_mxfp4_forward_ws(const void* x, const float* router_logits, const void* w13, const void* e13,
                         const void* w2, const void* e2, void* out, int M, int h, int i, int E, int k,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return run_forward_mx(x, router_logits, w13, e13, w2, e2, out, M, h, i, E, k, workspace, workspace_bytes,
                          stream);
}

int moe_mxfp4_forward_ws_timed(const void* x, const float* router_logits, const void* w13, const void* e13,
                               const void* w2, const void* e2, void* out, int M, int h, int i, int E, int k,
                               void* workspace, size_t workspace_bytes, hipEvent_t* events, int n_events,
                               hipStream_t stream) {
    if (!events) return MOE_ERR_INVALID;
    const int n = moe_mxfp4_forward_kernel_count(M, h, i, E, k);
    if (n < 0) return n;
    if (n_events < 2 * n) return MOE_ERR_INVALID;
    return run_forward_mx(x, router_logits, w13, e13, w2, e2, out, M, h, i, E, k, workspace, workspace_bytes,
                          stream, 1 << 30, events, n_events);
}

int moe_mxfp4_forward_ws_prefix(const void* x, const float* router_logits, const void* w13, const void* e13,
                                const void* w2, const void* e2, void* out, int M, int h, int i, int E, int k,
                                void* workspace, size_t workspace_bytes, int n_stages, hipStream_t stream) {
    if (n_stages < 0) return MOE_ERR_INVALID;
    return run_forward_mx(x, router_logits, w13, e13, w2, e2, out, M, h, i, E, k, workspace, workspace_bytes,
                          stream, n_stages);
}

const char* moe_fp8_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

int moe_fp8_workspace_layout(int M, int h, int i, int E, int k, moe_fp8_ws_layout* layout) {
    if (!layout) return MOE_ERR_INVALID;
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    Layout L;
    make_layout(M, h, i, E, k, &L);
    *layout = L.pub;
    return MOE_OK;
}

size_t moe_fp8_workspace_bytes_path(int M, int h, int i, int E, int k, int path) {
    if (M == 0 || check_shape(M, h, i, E, k) != MOE_OK || !path_ok(path, M, h, i, E, k, false)) return 0;
    Layout L;
    make_layout(M, h, i, E, k, &L, false, path);
    return L.pub.total;
}

int moe_fp8_workspace_layout_path(int M, int h, int i, int E, int k, int path, moe_fp8_ws_layout* layout) {
    if (!layout) return MOE_ERR_INVALID;
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (!path_ok(path, M, h, i, E, k, false)) return MOE_ERR_UNSUPPORTED;
    Layout L;
    make_layout(M, h, i, E, k, &L, false, path);
    *layout = L.pub;
    return MOE_OK;
}

int moe_fp8_forward_ws_path(const void* x, const float* router_logits, const void* w13, const float* s13,
                            const void* w2, const float* s2, void* out, int M, int h, int i, int E, int k,
                            void* workspace, size_t workspace_bytes, int path, hipStream_t stream) {
    if (path < 0) return MOE_ERR_INVALID;
    return run_forward(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, workspace, workspace_bytes,
                       nullptr, 0, stream, 1 << 30, path);
}

size_t moe_fp8_workspace_bytes(int M, int h, int i, int E, int k) {
    if (M == 0 || check_shape(M, h, i, E, k) != MOE_OK) return 0;
    Layout L;
    make_layout(M, h, i, E, k, &L);
    return L.pub.total;
}

int moe_fp8_bind_workspace(void* dev_ptr, size_t bytes) {
    if (dev_ptr && ((uintptr_t)dev_ptr % kAlign) != 0) return MOE_ERR_INVALID;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    if (dev_ptr && bytes < moe::kWorkspaceHead) return MOE_ERR_WORKSPACE;
    if (dev_ptr && hipMemset(dev_ptr, 0, moe::kWorkspaceHead) != hipSuccess) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_bind_mu);
    g_bind[dev].ptr = dev_ptr;
    g_bind[dev].bytes = dev_ptr ? bytes : 0;
    return MOE_OK;
}

int moe_fp8_forward_ws(const void* x, const float* router_logits, const void* w13,
                       const float* s13, const void* w2, const float* s2, void* out, int M, int h,
                       int i, int E, int k, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    return run_forward(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, workspace,
                       workspace_bytes, nullptr, 0, stream);
}

int moe_fp8_forward_ws_timed(const void* x, const float* router_logits, const void* w13,
                             const float* s13, const void* w2, const float* s2, void* out, int M,
                             int h, int i, int E, int k, void* workspace, size_t workspace_bytes,
                             hipEvent_t* events, int n_events, hipStream_t stream) {
    if (!events) return MOE_ERR_INVALID;
    const int n = moe_fp8_forward_kernel_count(M, h, i, E, k);
    if (n < 0) return n;
    if (n_events < 2 * n) return MOE_ERR_INVALID;
    return run_forward(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, workspace,
                       workspace_bytes, events, n_events, stream);
}

int moe_fp8_forward_ws_prefix(const void* x, const float* router_logits, const void* w13,
                              const float* s13, const void* w2, const float* s2, void* out, int M,
                              int h, int i, int E, int k, void* workspace, size_t workspace_bytes,
                              int n_stages, hipStream_t stream) {
    const int n = moe_fp8_forward_kernel_count(M, h, i, E, k);
    if (n < 0) return n;
    if (n_stages < 0 || n_stages > n) return MOE_ERR_INVALID;
    return run_forward(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, workspace,
                       workspace_bytes, nullptr, 0, stream, n_stages);
}

int moe_fp8_forward_kernel_count(int M, int h, int i, int E, int k) {
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return 0;
    return stage_count(choose_path(M, h, i, E, k), M, k);
}

const char* moe_fp8_forward_kernel_name(int M, int h, int i, int E, int k, int j) {
    const int n = moe_fp8_forward_kernel_count(M, h, i, E, k);
    if (n <= 0 || j < 0 || j >= n) return nullptr;
    return stage_name(choose_path(M, h, i, E, k), M, k, j);
}

size_t moe_fp8_workspace_head_bytes(void) { return moe::kWorkspaceHead; }

int moe_fp8_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!workspace || ((uintptr_t)workspace % kAlign) != 0) return MOE_ERR_INVALID;
    if (workspace_bytes < moe::kWorkspaceHead) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_zero_words(static_cast<uint32_t*>(workspace),
                                             moe::kWorkspaceHead / 4, stream));
}

int moe_fp8_workspace_status(void* workspace, size_t workspace_bytes, int clear, uint32_t* flags,
                             hipStream_t stream) {
    if (!workspace || !flags || ((uintptr_t)workspace % kAlign) != 0) return MOE_ERR_INVALID;
    if (workspace_bytes < moe::kWorkspaceHead) return MOE_ERR_WORKSPACE;
    uint32_t* word = at<uint32_t>(workspace, moe::kSyncErr);
    if (hipMemcpyAsync(flags, word, 4, hipMemcpyDeviceToHost, stream) != hipSuccess) return MOE_ERR_HIP;
    if (clear && moe::launch_zero_words(word, 1, stream) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(hipStreamSynchronize(stream));
}

int moe_fp8_probe_empty(int grid, hipStream_t stream) {
    if (grid < 1 || grid > (1 << 20)) return MOE_ERR_INVALID;
    return hip_status(moe::launch_probe_empty(grid, stream));
}

int moe_fp8_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream) {
    if (!src || !sink || !aligned16(src) || bytes % 16 != 0 || grid < 1 || grid > (1 << 20))
        return MOE_ERR_INVALID;
    if (bytes == 0) return MOE_OK;
    return hip_status(moe::launch_probe_read(src, bytes, grid, sink, stream));
}

int moe_fp8_forward_noalloc(const void* x, const float* router_logits, const void* w13, const float* s13,
                            const void* w2, const float* s2, void* out, int M, int h, int i, int E, int k,
                            hipStream_t stream) {
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return MOE_OK;
    if (!x || !router_logits || !w13 || !s13 || !w2 || !s2 || !out) return MOE_ERR_INVALID;
    Layout L;
    make_layout(M, h, i, E, k, &L);
    if (L.pub.total > kScratchBytes) return MOE_ERR_WORKSPACE;   // beyond the fixed array
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            // first call on this device (which is current): the array's
            // device address, checked; its synchronisation head is zero from
            // the module load and is cleared once more by a fill kernel ahead
            // of this forward unless the stream is being captured (a
            // captured clear would rerun on every replay)
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MOE_ERR_HIP;
            if (cs == hipStreamCaptureStatusNone &&
                moe::launch_zero_words(static_cast<uint32_t*>(p), moe::kWorkspaceHead / 4, stream) != hipSuccess)
                return MOE_ERR_HIP;
            g_scratch_ptr[dev] = p;
        }
        ws = g_scratch_ptr[dev];
    }
    return run_forward(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, ws, kScratchBytes, nullptr, 0,
                       stream);
}

int moe_fp8_forward(const void* x, const float* router_logits, const void* w13, const float* s13,
                    const void* w2, const float* s2, void* out, int M, int h, int i, int E, int k,
                    hipStream_t stream) {
    const int rc = check_shape(M, h, i, E, k);
    if (rc != MOE_OK) return rc;
    if (M == 0) return MOE_OK;
    if (!x || !router_logits || !w13 || !s13 || !w2 || !s2 || !out) return MOE_ERR_INVALID;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    Binding b;
    {
        std::lock_guard<std::mutex> lock(g_bind_mu);
        b = g_bind[dev];
    }
    if (!b.ptr) return MOE_ERR_WORKSPACE;
    return moe_fp8_forward_ws(x, router_logits, w13, s13, w2, s2, out, M, h, i, E, k, b.ptr, b.bytes,
                              stream);
}

int router_topk(const float* logits, int M, int E, int k, int32_t* topk_ids, float* topk_w,
                hipStream_t stream) {
    if (M < 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID;
    if (E > MOE_FP8_MAX_EXPERTS || k > MOE_FP8_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID;
    return hip_status(moe::launch_route_quant(logits, nullptr, M, E, k, 128, topk_ids, topk_w,
                                              nullptr, nullptr, moe::kRoute, stream));
}

int moe_fp8_router_gemm_topk(const void* x, const void* wr, int M, int h, int E, int k, float* logits,
                             int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    if (M < 0 || h <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID;
    if (h % 128 != 0 || h > MOE_FP8_MAX_HIDDEN || E > MOE_FP8_MAX_EXPERTS || k > MOE_FP8_MAX_TOPK || k > E)
        return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !wr || !topk_ids || !topk_w) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(wr)) return MOE_ERR_INVALID;
    return hip_status(moe::launch_router_gemm_topk(static_cast<const uint16_t*>(x),
                                                   static_cast<const uint16_t*>(wr), M, h, E, k, logits,
                                                   topk_ids, topk_w, stream));
}

int moe_fp8_act_quant(const void* x, int M, int K, uint8_t* q, float* s, hipStream_t stream) {
    if (M < 0 || K <= 0) return MOE_ERR_INVALID;
    if (K % 128 != 0 || K > MOE_FP8_MAX_HIDDEN) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !q || !s) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(q)) return MOE_ERR_INVALID;
    return hip_status(moe::launch_route_quant(nullptr, static_cast<const uint16_t*>(x), M, 1, 1, K,
                                              nullptr, nullptr, q, s, moe::kQuant, stream));
}

int moe_fp8_rmsnorm_act_quant(const void* x, const float* gamma, float eps, int M, int h, void* y,
                              uint8_t* q, float* s, hipStream_t stream) {
    if (M < 0 || h <= 0 || !(eps >= 0.0f) || eps > 3.0e38f) return MOE_ERR_INVALID;
    if (h % 128 != 0 || h > moe::kFrontMaxHidden) return MOE_ERR_UNSUPPORTED;
    if (M == 0) return MOE_OK;
    if (!x || !gamma || !q || !s) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(q) || !aligned16(s) || (y && !aligned16(y)))
        return MOE_ERR_INVALID;
    return hip_status(moe::launch_rmsnorm_quant(static_cast<const uint16_t*>(x), gamma, eps, M, h,
                                                static_cast<uint16_t*>(y), q, s, stream));
}

size_t moe_fp8_group_workspace_bytes(int M, int E, int k) {
    if (M < 0 || E <= 0 || k <= 0 || E > MOE_FP8_MAX_EXPERTS) return 0;
    return align_up((size_t)moe::group_chunks(M * k) * E * 4 + 2 * (size_t)E * 4 + 64);
}

int moe_fp8_group(const int32_t* topk_ids, int M, int E, int k, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_route_ids, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    if (M < 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID;
    if (E > MOE_FP8_MAX_EXPERTS || k > MOE_FP8_MAX_TOPK || k > E) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)M * k > (int64_t)1 << 28) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID;
    if (M > 0 && (!topk_ids || !sorted_route_ids)) return MOE_ERR_INVALID;
    if (!workspace || workspace_bytes < moe_fp8_group_workspace_bytes(M, E, k))
        return MOE_ERR_WORKSPACE;
    const int R = M * k;
    int32_t* hist = static_cast<int32_t*>(workspace);
    int32_t* active = hist + (size_t)moe::group_chunks(R) * E;
    int32_t* num_active = active + E;
    return hip_status(moe::launch_group(topk_ids, R, E, hist, counts, offsets, sorted_route_ids,
                                        active, num_active, stream));
}

int moe_fp8_quantize_weight_block128(const float* w, int64_t batch, int N, int K, uint8_t* q,
                                     float* s, hipStream_t stream) {
    if (batch < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID;
    if (N % 128 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (batch == 0) return MOE_OK;
    if (!w || !q || !s || !aligned16(w) || !aligned16(q)) return MOE_ERR_INVALID;
    return hip_status(moe::launch_quant_weight(w, batch, N, K, q, s, stream));
}

int moe_fp8_encode_e4m3(const float* in, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n < 0) return MOE_ERR_INVALID;
    if (n == 0) return MOE_OK;
    if (!in || !out) return MOE_ERR_INVALID;
    return hip_status(moe::launch_encode_e4m3(in, n, out, stream));
}

}  // extern "C"
