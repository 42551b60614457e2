// group.hip -- deterministic grouping of the M*k routes by expert
// (Netra Kernel README, MoE prefill pair: the metadata stage; Inferact
// amd-kernels README, atomics rule: atomics may count, never decide order).
//
// Pass 1: one workgroup per chunk of 256 routes counts routes per expert
// with LDS atomic increments (an integer count does not depend on their
// order).
// Pass 2: one workgroup per chunk sums every expert's chunk counts (1024
// threads read the chunk histograms in parallel: all chunks for the totals,
// the earlier ones for this chunk's start), then one wave derives the global
// offsets by a prefix sum and scatters the chunk's routes in route order, 64
// at a time: a lane's rank among equal experts in its batch comes from a
// ballot match over the 9 bits of the expert id, so the sorted order is route
// id ascending inside each expert by construction.
// Chunk 0 also writes counts, offsets, the ascending list of experts that
// received routes and, when asked, each expert's first M-tile index for a
// grouped GEMM with tile_m routes per tile (exclusive scan of
// ceil(count / tile_m)).
#include "device.h"
#include "group.h"
#include "launch.h"

namespace moe {

constexpr int kChunk = 256;     // routes per chunk: one workgroup of each pass per chunk
constexpr int kScanGroups = 4;  // chunk-histogram readers per expert in pass 2 (1024 threads)

int group_chunks(int R) { return R <= 0 ? 1 : (R + kChunk - 1) / kChunk; }

// E <= 256: thread t counts into bin t.
__global__ __launch_bounds__(kChunk) void group_hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                            int32_t* __restrict__ hist) {
    __shared__ int cnt[256];
    const int t = threadIdx.x;
    cnt[t] = 0;
    __syncthreads();
    const int beg = blockIdx.x * kChunk;
    group_chunk_hist(ids, beg, min(R, beg + kChunk), E, cnt, t, kChunk);
    __syncthreads();
    if (t < E) hist[(size_t)blockIdx.x * E + t] = cnt[t];
}

__global__ __launch_bounds__(256 * kScanGroups) void group_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nchunks, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active, int tile_m,
    int32_t* __restrict__ mtile_off) {
    __shared__ int tot_l[kScanGroups * 256], pre_l[kScanGroups * 256];
    __shared__ int base_l[256];
    const int chunk = blockIdx.x, beg = chunk * kChunk;
    const GroupOut o{counts, offsets, sorted, active, num_active, tile_m > 0 ? mtile_off : nullptr, tile_m};
    group_chunk_scatter<kScanGroups>(ids, E, nchunks, hist, chunk, beg, min(R, beg + kChunk), chunk == 0, o, tot_l,
                                     pre_l, base_l, threadIdx.x);
}

hipError_t launch_group(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, int32_t* active, int32_t* num_active,
                        hipStream_t stream, int tile_m, int32_t* mtile_off) {
    const int nchunks = group_chunks(R);
    launch(group_hist_kernel, dim3(nchunks), dim3(kChunk), 0, stream, ids, R, E, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    launch(group_scatter_kernel, dim3(nchunks), dim3(256 * kScanGroups), 0, stream, ids, R, E, nchunks,
                       hist, counts, offsets, sorted, active, num_active, tile_m, mtile_off);
    return hipGetLastError();
}

}  // namespace moe
