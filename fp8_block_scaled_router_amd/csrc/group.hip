// group.hip -- deterministic grouping of the M*k routes by expert
// (Netra Kernel README, MoE prefill pair: the metadata stage; Inferact
// amd-kernels README, atomics rule: atomics may count, never decide order).
//
// Pass 1: one workgroup per chunk of routes counts routes per expert with
// LDS atomic increments (an integer count does not depend on their order).
// Pass 2: one wave per chunk derives every expert's global offset and its
// chunk-local start from the chunk histograms, then scatters the chunk's
// routes in route order, 64 at a time (ids requested 16 batches ahead): a lane's rank among equal experts in
// its batch comes from a ballot match over the 9 bits of the expert id, so
// the sorted order is route id ascending inside each expert by construction.
// Chunk 0 also writes counts, offsets, the ascending list of experts that
// received routes and, when asked, each expert's first M-tile index for a
// grouped GEMM with tile_m routes per tile (exclusive scan of
// ceil(count / tile_m)).
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kChunk = 4096;

int group_chunks(int R) { return R <= 0 ? 1 : (R + kChunk - 1) / kChunk; }

__global__ __launch_bounds__(256) void group_hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                         int32_t* __restrict__ hist) {
    __shared__ int cnt[256];
    for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int beg = blockIdx.x * kChunk;
    const int end = min(R, beg + kChunk);
    for (int p = beg + threadIdx.x; p < end; p += 256) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // ids outside [0, E) are dropped
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = cnt[e];
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

__global__ __launch_bounds__(64) void group_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nchunks, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active, int tile_m,
    int32_t* __restrict__ mtile_off) {
    __shared__ int base[256];
    const int chunk = blockIdx.x;
    const int lane = threadIdx.x;
    // Lane l owns experts 4l .. 4l+3; the histograms of 8 chunks are
    // requested together, so the prefix costs one memory round trip per 8
    // chunks instead of one per chunk.
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
        int v[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 4 * lane + j, c = c0 + u;
                v[u][j] = (e < E && c < nchunks) ? hist[(size_t)c * E + e] : 0;
            }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (c0 + u < chunk) pre[j] += v[u][j];
                tot[j] += v[u][j];
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
    __syncthreads();

    const int beg = chunk * kChunk;
    const int end = min(R, beg + kChunk);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // the ids of 16 batches are requested together
    for (int q0 = beg; q0 < end; q0 += 16 * 64) {
        int ev[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int p = q0 + 64 * u + lane;
            ev[u] = p < end ? ids[p] : 0x1FF;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int p0 = q0 + 64 * u;
            if (p0 >= end) break;
            const int p = p0 + lane;
            int e = ev[u];
            const bool valid = (unsigned)e < (unsigned)E;
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
            int pos = 0;
            if (valid) pos = base[e] + rank;
            __syncthreads();
            if (valid) {
                sorted[pos] = p;
                if (last) base[e] += __popcll(same);
            }
            __syncthreads();
        }
    }
}

hipError_t launch_group(const int32_t* ids, int R, int E, int32_t* hist, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, int32_t* active, int32_t* num_active,
                        hipStream_t stream, int tile_m, int32_t* mtile_off) {
    const int nchunks = group_chunks(R);
    hipLaunchKernelGGL(group_hist_kernel, dim3(nchunks), dim3(256), 0, stream, ids, R, E, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(group_scatter_kernel, dim3(nchunks), dim3(64), 0, stream, ids, R, E, nchunks,
                       hist, counts, offsets, sorted, active, num_active, tile_m, mtile_off);
    return hipGetLastError();
}

}  // namespace moe
