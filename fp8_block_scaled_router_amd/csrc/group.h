// group.h -- the grouping of one chunk of routes by expert as device
// functions, shared by the grouping launches (group.hip) and the prefill
// producer.  A chunk counts its routes per expert (group_chunk_hist); once
// every chunk's counts are in `hist`, each chunk sums every expert's counts
// over all chunks and over the chunks before it, derives the offsets by a
// prefix sum, and scatters its own routes in route order (group_chunk_scatter).
#pragma once

#include "device.h"

namespace moe {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Outputs of the grouping (written by the chunk that is asked to).
struct GroupOut {
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* num_active;
    int32_t* mtile_off;   // null: not wanted
    int tile_m;
};

// Counts of routes beg .. end - 1 per expert into cnt[0 .. E) (LDS, cleared
// by the caller; ids outside [0, E) are dropped); threads t, t + nt, ...
__device__ __forceinline__ void group_chunk_hist(const int32_t* __restrict__ ids, int beg, int end, int E, int* cnt,
                                                 int t, int nt) {
    for (int p = beg + t; p < end; p += nt) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
}

// Plain or device-scope (kCoh: across the workgroups of one launch) int
// accesses.
template <bool kCoh>
__device__ __forceinline__ int ld_i32(const int32_t* p) {
    if constexpr (kCoh) return (int)ld_agent(reinterpret_cast<const uint32_t*>(p));
    else return *p;
}
template <bool kCoh>
__device__ __forceinline__ void st_i32(int32_t* p, int v) {
    if constexpr (kCoh) st_agent(reinterpret_cast<uint32_t*>(p), (uint32_t)v);
    else *p = v;
}

// Grouping of chunk `chunk` (routes beg .. end - 1) of nchunks, whose rows of
// E counts are in hist; NG * 256 threads.  Thread (g, e) sums expert e's
// counts over chunks g, g + NG, ... (all of them, and those before this
// chunk), kBatch requests at a time, into tot_l / pre_l (NG * 256 ints each, LDS
// scratch); then wave 0 derives the offsets (base_l: 256 ints) and scatters
// the chunk's routes in route order, 64 at a time: a lane's rank among equal
// experts in its batch comes from a ballot match over the 9 bits of the
// expert id, so the sorted order is route id ascending inside each expert by
// construction.  With `writer` set the chunk also writes counts, offsets, the
// ascending list of experts that received routes and, when asked, each
// expert's first M-tile index for tiles of tile_m routes (exclusive scan of
// ceil(count / tile_m)).  The caller synchronises the workgroup afterwards.
// kCoh: hist is read, and the outputs written, at device scope (within one
// launch, across workgroups); kBatch: loads in flight per thread and round.
template <int NG, bool kCoh = false, int kBatch = 16>
__device__ __forceinline__ void group_chunk_scatter(const int32_t* __restrict__ ids, int E, int nchunks,
                                                    const int32_t* __restrict__ hist, int chunk, int beg, int end,
                                                    bool writer, const GroupOut& o, int* tot_l, int* pre_l,
                                                    int* base_l, int tid) {
    {
        const int e = tid & 255, g = tid >> 8;
        int tot = 0, pre = 0;
        if (e < E) {
            for (int c0 = g; c0 < nchunks; c0 += kBatch * NG) {
                int v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int c = c0 + NG * u;
                    v[u] = c < nchunks ? ld_i32<kCoh>(hist + (size_t)c * E + e) : 0;
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    tot += v[u];
                    if (c0 + NG * u < chunk) pre += v[u];
                }
            }
        }
        tot_l[g * 256 + e] = tot;
        pre_l[g * 256 + e] = pre;
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
        for (int g = 0; g < NG; ++g) {
            tot[j] += tot_l[g * 256 + e];
            pre[j] += pre_l[g * 256 + e];
        }
    }
    const int lsum = tot[0] + tot[1] + tot[2] + tot[3];
    const int lact = (tot[0] > 0) + (tot[1] > 0) + (tot[2] > 0) + (tot[3] > 0);
    int ltiles = 0;
    if (o.mtile_off)
        for (int j = 0; j < 4; ++j) ltiles += (tot[j] + o.tile_m - 1) / o.tile_m;
    const int incl = wave_incl_scan(lsum, lane);
    const int iact = wave_incl_scan(lact, lane);
    const int itil = wave_incl_scan(ltiles, lane);
    int run = incl - lsum, arun = iact - lact, trun = itil - ltiles;
    if (writer && o.mtile_off) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            if (e < E) st_i32<kCoh>(o.mtile_off + e, trun);
            trun += (tot[j] + o.tile_m - 1) / o.tile_m;
        }
        if (lane == 63) st_i32<kCoh>(o.mtile_off + E, itil);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        if (e < E) {
            base_l[e] = run + pre[j];
            if (writer) {
                st_i32<kCoh>(o.offsets + e, run);
                st_i32<kCoh>(o.counts + e, tot[j]);
                if (tot[j] > 0) st_i32<kCoh>(o.active + arun, e);
            }
        }
        run += tot[j];
        arun += (tot[j] > 0);
    }
    if (writer && lane == 63) {
        st_i32<kCoh>(o.offsets + E, incl);
        st_i32<kCoh>(o.num_active, iact);
    }

    // Scatter the chunk's routes in route order, 64 at a time (one wave, so
    // the LDS reads and updates of base_l stay in program order).
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int b0 = beg; b0 < end; b0 += 4 * 64) {
        int ev[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = b0 + 64 * u + lane;
            ev[u] = p < end ? ids[p] : 0x1FF;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = b0 + 64 * u + lane;
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
            const int pos = valid ? base_l[e] + rank : 0;
            if (valid) {
                st_i32<kCoh>(o.sorted + pos, p);
                if (last) base_l[e] += __popcll(same);
            }
        }
    }
}

}  // namespace moe
