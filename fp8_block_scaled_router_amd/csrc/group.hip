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
    const int p = blockIdx.x * kChunk + t;
    if (p < R) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // ids outside [0, E) are dropped
    }
    __syncthreads();
    if (t < E) hist[(size_t)blockIdx.x * E + t] = cnt[t];
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__global__ __launch_bounds__(256 * kScanGroups) void group_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nchunks, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active, int tile_m,
    int32_t* __restrict__ mtile_off) {
    __shared__ int tot_l[kScanGroups][256], pre_l[kScanGroups][256];
    __shared__ int base[256];
    const int chunk = blockIdx.x;
    const int tid = threadIdx.x;
    {
        // Thread (g, e) sums expert e's counts over chunks g, g + 4, ...
        // (all of them, and those before this chunk), 16 requests at a time.
        const int e = tid & 255, g = tid >> 8;
        int tot = 0, pre = 0;
        if (e < E) {
            for (int c0 = g; c0 < nchunks; c0 += 16 * kScanGroups) {
                int v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int c = c0 + kScanGroups * u;
                    v[u] = c < nchunks ? hist[(size_t)c * E + e] : 0;
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    tot += v[u];
                    if (c0 + kScanGroups * u < chunk) pre += v[u];
                }
            }
        }
        tot_l[g][e] = tot;
        pre_l[g][e] = pre;
    }
    __syncthreads();
    if (tid >= kWave) return;
    // One wave from here on; lane l owns experts 4l .. 4l+3.
    const int lane = tid;
    int tot[4], pre[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        tot[j] = 0;
        pre[j] = 0;
#pragma unroll
        for (int g = 0; g < kScanGroups; ++g) {
            tot[j] += tot_l[g][e];
            pre[j] += pre_l[g][e];
        }
    }
    const int lsum = tot[0] + tot[1] + tot[2] + tot[3];
    const int lact = (tot[0] > 0) + (tot[1] > 0) + (tot[2] > 0) + (tot[3] > 0);
    int ltiles = 0;
    if (tile_m > 0)
        for (int j = 0; j < 4; ++j) ltiles += (tot[j] + tile_m - 1) / tile_m;
    const int incl = wave_incl_scan(lsum, lane);
    const int iact = wave_incl_scan(lact, lane);
    const int itil = wave_incl_scan(ltiles, lane);
    int run = incl - lsum, arun = iact - lact, trun = itil - ltiles;
    if (chunk == 0 && tile_m > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            if (e < E) mtile_off[e] = trun;
            trun += (tot[j] + tile_m - 1) / tile_m;
        }
        if (lane == 63) mtile_off[E] = itil;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        if (e < E) {
            base[e] = run + pre[j];
            if (chunk == 0) {
                offsets[e] = run;
                counts[e] = tot[j];
                if (tot[j] > 0) active[arun] = e;
            }
        }
        run += tot[j];
        arun += (tot[j] > 0);
    }
    if (chunk == 0 && lane == 63) {
        offsets[E] = incl;
        *num_active = iact;
    }

    // Scatter the chunk's routes in route order, 64 at a time (one wave, so
    // the LDS reads and updates of base stay in program order).
    const int beg = chunk * kChunk;
    const int end = min(R, beg + kChunk);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int ev[kChunk / 64];
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) {
        const int p = beg + 64 * u + lane;
        ev[u] = p < end ? ids[p] : 0x1FF;
    }
#pragma unroll
    for (int u = 0; u < kChunk / 64; ++u) {
        const int p = beg + 64 * u + lane;
        int e = ev[u];
        const bool valid = p < end && (unsigned)e < (unsigned)E;
        if (!valid) e = 0x1FF;
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & below);
        const bool last = (same >> lane) == 1ull;   // highest lane of its expert in this batch
        const int pos = valid ? base[e] + rank : 0;
        if (valid) {
            sorted[pos] = p;
            if (last) base[e] += __popcll(same);
        }
    }
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
