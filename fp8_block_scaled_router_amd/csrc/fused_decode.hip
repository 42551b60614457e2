// fused_decode.hip -- the whole layer in one kernel for one or two tokens
// (decode).
//
// The work is cut along the expert intermediate dimension.  A unit is
// (active expert slot u, 128-column block ib of the intermediate); P
// workgroups (parts, P = 8 or 4) share each unit.  Part q of unit (u, ib)
// owns
//   - 128/P gate rows ib*128 + q*128/P .. of w13[e_u] and the matching up
//     rows, over K = h: the gate/up GEMM of those columns (Netra compiler
//     architecture page: gate/up with FP32 results), K blocks split over the
//     four waves;
//   - rows q*h/P .. (q+1)*h/P of w2[e_u], columns ib*128 .. +128: one 128-wide
//     K block of the down GEMM for those output rows.
// Because the SiLU-mul requantisation groups are exactly the 128-column
// blocks of the intermediate (the 1x128 activation quantisation of the down
// GEMM's input), a unit's down-partial needs only the unit's own gate/up
// columns.  So as soon as a workgroup knows its expert it requests its w13
// rows into registers, and its w2 rows right after its gate/up MFMAs: the
// w13 requests of the whole layer go out first, the w2 stream overlaps the
// exchange of the SiLU-mul values, and no workgroup waits for another before
// its weights arrive.
//
// Exchanges between workgroups (each value one 64-bit word: value | tag of
// this forward, written and read with agent-scope relaxed atomics; the data
// is its own flag):
//   v  [route][i]      SiLU(gate) * up of each part's columns; every part of
//                      the unit reads all 128 of its block, takes amax/448 and
//                      the E4M3 codes itself (identical inputs, identical
//                      codes), then multiplies its w2 rows.
//   t  [route][ib][h]  the down GEMM's block terms blk * (a2s * s2): the K
//                      block ib's contribution to the partial of each route.
// Combine (route reducer; Inferact amd-kernels README, atomics rule: a fixed
// order, no atomic adds): per 64 output columns, y_r = sum of t over the
// blocks ib ascending (the down GEMM's per-block accumulation order), then
// out = bf16(sum over ranks r ascending of w_r * y_r).
//
// Every workgroup first recomputes what it needs from the batch: the router
// top-k of all M tokens (one wave per token), the active experts, the
// grouping of the routes, and the 1x128 E4M3 activation codes of all tokens
// (into LDS).  Waits are bounded in time: a wait that times out sets the
// workspace's sticky error word and the late value is replaced by NaN, which
// reaches the output.  Every awaited value is produced by a workgroup that is
// resident at the same time (the grid never exceeds the resident capacity)
// and that waits on nothing but its unit's peers before producing it.  The
// last workgroup to exit advances the forward tag.
#include "device.h"
#include "fused_decode.h"
#include "launch.h"

namespace moe {

constexpr int kFusedMaxM = 4;
constexpr int kFusedMaxIB = 8;              // i <= 1024
constexpr int kFusedMaxKB = 16;             // h <= 2048
constexpr int kFusedMaxGrid = 512;          // two workgroups per CU on 256 CUs
constexpr int kKBW = kFusedMaxKB / 4;       // K blocks of gate/up per wave
constexpr uint64_t kWaitTicks = 100000000;  // 1 s of the 100 MHz constant clock

__device__ __forceinline__ uint32_t readlane_u(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint32_t row16_min_u(uint32_t v) {
    v = min(v, dpp_u<kDppQuadXor1>(v));
    v = min(v, dpp_u<kDppQuadXor2>(v));
    v = min(v, dpp_u<kDppRowHalfMirror>(v));
    v = min(v, dpp_u<kDppRowMirror>(v));
    return v;
}
// Unsigned max / min over the wave: DPP inside each row of 16, then the two
// gfx950 row swaps; every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
    v = row16_max_u(v);
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(p[0], p[1]);
    p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(p[0], p[1]);
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
    v = row16_min_u(v);
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min(p[0], p[1]);
    p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return min(p[0], p[1]);
}

// Router of one token on one wave; lane l holds the logits of experts
// l + 64j as order keys (0 = no expert).  Each pick is branch-free: the wave
// max of the keys, then the wave min of the expert index among the keys that
// reach it (ties go to the lower index, -0 equals +0), which is knocked out.
// Lane r keeps pick r; the weights exp(l_r - l_0) / sum are summed in rank
// order.  route_rounds(s, r0, r1) makes picks r0 .. r1 - 1, so a caller can
// act on the first picks before making the rest.
struct RouteState {
    uint32_t key[4];
    uint32_t pick, pkey;   // lane r: pick r and its key
};

__device__ __forceinline__ void route_begin(RouteState& s, const float lg[4], int E, int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s.key[j] = (lane + 64 * j < E) ? float_order_key(lg[j]) : 0u;
    s.pick = 0u;
    s.pkey = 0u;
}

__device__ __forceinline__ void route_rounds(RouteState& s, int r0, int r1, int E, int lane) {
#pragma unroll 1
    for (int r = r0; r < r1; ++r) {
        const uint32_t m = wave_max_u(max(max(s.key[0], s.key[1]), max(s.key[2], s.key[3])));
        const uint32_t cand = s.key[0] == m ? (uint32_t)lane
                            : s.key[1] == m ? (uint32_t)(64 + lane)
                            : s.key[2] == m ? (uint32_t)(128 + lane)
                            : s.key[3] == m ? (uint32_t)(192 + lane) : 0x1FFu;
        uint32_t e = wave_min_u(cand);
        e = (m == 0u || e >= (uint32_t)E) ? (uint32_t)(E - 1) : e;   // only for NaN logits (outside the contract)
#pragma unroll
        for (int j = 0; j < 4; ++j) s.key[j] = (uint32_t)(lane + 64 * j) == e ? 0u : s.key[j];
        s.pick = lane == r ? e : s.pick;
        s.pkey = lane == r ? m : s.pkey;
    }
}

__device__ __forceinline__ void route_end(const RouteState& s, int k, int* ids_l, float* w_l, int lane) {
    const float l0 = float_from_order_key(readlane_u(s.pkey, 0));
    const float ex = lane < k ? expf(float_from_order_key(s.pkey) - l0) : 0.0f;
    float sum = 0.0f;
#pragma unroll 1
    for (int r = 0; r < k; ++r) sum += __uint_as_float(readlane_u(__float_as_uint(ex), r));
    if (lane < k) {
        ids_l[lane] = (int)s.pick;
        w_l[lane] = ex / sum;
    }
}

__device__ __forceinline__ void route_fast(const float lg[4], int E, int k, int* ids_l,
                                           float* w_l, int lane) {
    RouteState s;
    route_begin(s, lg, E, lane);
    route_rounds(s, 0, k, E, lane);
    route_end(s, k, ids_l, w_l, lane);
}

// Lanes holding the same expert id (9-bit ids; 0x1FF = no route).
__device__ __forceinline__ uint64_t match_id(int e) {
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    return same;
}

// Waiting on words that other workgroups write.  Heavy polling of a line
// slows the stores that other CUs direct at it (measured: with every lane of
// many workgroups re-reading all of its words, a producer's stores stalled
// until the pollers gave up), so a wait first polls one sentinel word per
// producer -- the last word that producer writes into the range -- with one
// load per lane and a short sleep between rounds (two rounds of s_sleep 2 at
// most: longer sleeps add their length to the hand-off, shorter ones slow the
// producers' stores; measured), then reads the data once and re-reads only
// while some word still lacks the tag.

// Lane-wise: loads *p until it carries `tag` (lanes with p == nullptr are
// done at once).  Returns false when the wait timed out (the sticky error
// word is then set).
__device__ __forceinline__ bool wait_sentinel(const uint64_t* p, uint32_t tag, uint32_t* err) {
    uint64_t t0 = 0;
    int nap = 1;
    for (int tries = 0;; ++tries) {
        const bool ok = p == nullptr || ll_tag(ld_agent64(p)) == tag;
        if (__ballot(!ok) == 0ull) return true;
        if (tries == 0) t0 = wall_clock64();
        if (wall_clock64() - t0 > kWaitTicks) {
            atomicOr(err, 1u);
            return false;
        }
        for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
        nap = nap < 2 ? 2 * nap : 2;
    }
}

// Loads the tagged words p[0..N) (issued together, no conditions; every
// pointer must address a word written in this forward) until each carries
// `tag`.  Returns false when the wait timed out.
template <int N>
__device__ __forceinline__ bool read_words(const uint64_t* const (&p)[N], uint32_t tag, uint64_t (&w)[N],
                                           uint32_t* err) {
    uint64_t t0 = 0;
    for (int tries = 0;; ++tries) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < N; ++j) w[j] = ld_agent64(p[j]);
#pragma unroll
        for (int j = 0; j < N; ++j) ok = ok && ll_tag(w[j]) == tag;
        if (__ballot(!ok) == 0ull) return true;
        if (tries == 0) t0 = wall_clock64();
        if (wall_clock64() - t0 > kWaitTicks) {
            atomicOr(err, 1u);
            return ok;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// LDS carve of one workgroup (all offsets 16-byte aligned).
struct FusedLds {
    size_t xq, xs, ids, w, off, act, srt, cnt, misc, sc2, blk, a2, a2s, y, bounce, total;
};

__host__ __device__ inline size_t r16(size_t v) { return (v + 15) & ~(size_t)15; }

template <int P, int MM>
__host__ __device__ inline FusedLds fused_lds(int M, int h, int E, int k) {
    constexpr int NT = 128 / P / 16;
    const int R = M * k;
    FusedLds L;
    size_t o = 0;
    L.xq = o;     o += r16((size_t)M * h);
    L.xs = o;     o += (size_t)M * kFusedMaxKB * 4;   // one 16-float row per token
    L.ids = o;    o += r16((size_t)R * 4);
    L.w = o;      o += r16((size_t)R * 4);
    L.off = o;    o += r16((size_t)(E + 1) * 4);
    L.act = o;    o += r16((size_t)E * 4);
    L.srt = o;    o += r16((size_t)R * 4);
    L.cnt = o;    o += r16((size_t)E * 4);
    L.misc = o;   o += 32 * 4;
    L.sc2 = o;    o += 16 * 4;
    L.blk = o;    o += (size_t)2 * NT * kFusedMaxKB * 16 * MM * 4;
    L.a2 = o;     o += (size_t)MM * 128;
    L.a2s = o;    o += 16;
    L.y = o;      o += (size_t)16 * 64 * 4;
    L.bounce = o; o += (size_t)4 * 2 * 2048;
    L.total = o;
    return L;
}

template <int P, int MM>
__global__ __launch_bounds__(256) void fused_decode_kernel(FusedArgs a) {
    constexpr int NT = 128 / P / 16;            // 16-row tiles of gate (and of up) per part
    // w2 tiles go to waves kDW0..3: with P = 8 wave 0 holds none, so that its
    // loads of the exchanged values (the vector memory counter retires in
    // issue order) never wait behind the w2 stream.
    constexpr int kDW0 = P == 8 ? 1 : 0;
    constexpr int kDWN = 4 - kDW0;
    constexpr int NDT = (2048 / P / 16 + kDWN - 1) / kDWN;   // down tiles per wave at h = 2048
    extern __shared__ __align__(16) uint8_t smem[];
    const int M = a.M, h = a.h, i = a.i, E = a.E, k = a.k;
    const int R = M * k, G = h / 128, IB = i / 128, KB = h / 128, N13 = 2 * i;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    uint32_t* err = a.sync + kSyncErr / 4;
    const int q = blockIdx.x % P, uid = blockIdx.x / P;
    const int u = uid / IB, ib = uid - u * IB;
    const int drows = h / P, ndt = drows / 16;   // this part's w2 rows and their 16-row tiles
    const int nb0 = (q * drows) / 128;           // first 128-row block of those rows

    const FusedLds Lo = fused_lds<P, MM>(M, h, E, k);
    uint8_t* xq_l = smem + Lo.xq;                                   // [M][h]
    float* xs_l = reinterpret_cast<float*>(smem + Lo.xs);          // [M][kFusedMaxKB] (G used)
    int* ids_l = reinterpret_cast<int*>(smem + Lo.ids);            // [R]
    float* w_l = reinterpret_cast<float*>(smem + Lo.w);            // [R]
    int* off_l = reinterpret_cast<int*>(smem + Lo.off);            // [E+1]
    int* act_l = reinterpret_cast<int*>(smem + Lo.act);            // [E]
    int* srt_l = reinterpret_cast<int*>(smem + Lo.srt);            // [R]
    int* cnt_l = reinterpret_cast<int*>(smem + Lo.cnt);            // [E]
    int* misc_l = reinterpret_cast<int*>(smem + Lo.misc);          // [32]
    float* sc2_l = reinterpret_cast<float*>(smem + Lo.sc2);        // [16]
    float* blk_l = reinterpret_cast<float*>(smem + Lo.blk);        // [2NT][kFusedMaxKB][16][MM]
    uint8_t* a2_l = smem + Lo.a2;                                   // [MM][128]
    float* a2s_l = reinterpret_cast<float*>(smem + Lo.a2s);        // [MM]
    float* y_l = reinterpret_cast<float*>(smem + Lo.y);            // [16][64]
    uint8_t* bounce = smem + Lo.bounce + wave * 4096;               // [2][2048] per wave

    // The part's gate/up weights: block scales first, then w13 (the gate/up
    // tiles, this wave's K blocks kb = wave + 4j), each tile as whole 128-byte
    // lines (w2 follows after the gate/up MFMAs).  Unconditional loads (a K
    // block or tile past the end re-reads the last one and is not used): a
    // conditionally loaded register would be copied into place after its
    // load, which makes the wave wait for it.
    v8i A[2 * NT][kKBW];
    v8i D[NDT];
    float sc_v = 0.0f;
    auto issue_w13 = [&](int ex) {
        if (wave == 0) {
            if (lane < 2 * kFusedMaxKB && (lane & (kFusedMaxKB - 1)) < KB) {
                const int blk_row = lane < kFusedMaxKB ? ib : IB + ib;
                sc_v = a.s13[((size_t)ex * (N13 / 128) + blk_row) * KB + (lane & (kFusedMaxKB - 1))];
            } else if (lane >= 32 && lane - 32 <= (q * drows + drows - 1) / 128 - nb0) {
                sc_v = a.s2[((size_t)ex * (h / 128) + nb0 + lane - 32) * IB + ib];
            }
        }
#pragma unroll
        for (int t2 = 0; t2 < 2 * NT; ++t2) {
            const int row = (t2 < NT ? 0 : i) + ib * 128 + q * (128 / P) + (t2 % NT) * 16;
            const uint8_t* base = a.w13 + ((size_t)ex * N13 + row) * h;
#pragma unroll
            for (int j = 0; j < kKBW; ++j) A[t2][j] = load_lines_nt(base + min(wave + 4 * j, KB - 1) * 128, h, lane);
        }
    };

    // ---- phase 0: tag, routing of every token, active experts
    uint32_t epoch = 0u;
    if (tid == 0) epoch = ld_agent(a.sync + kSyncEpoch / 4);
    const int nq = M * G;   // 16-lane rows of activation groups (<= 64)
    const int qbase = wave * 4 + (lane >> 4);
    uint4 xr[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int task = min(qbase + 16 * s4, nq - 1);
        const int t = task / G, g = task - t * G;
        xr[s4] = *reinterpret_cast<const uint4*>(a.x + (size_t)t * h + g * 128 + col * 8);
    }
    float lg[4];
    auto l_load = [&](int t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            lg[j] = (t < M && e < E) ? a.logits[(size_t)t * E + e] : 0.0f;
        }
    };
    int e_rank = 0;
    if constexpr (MM == 1) {
        // One token: with the active experts numbered in rank order, unit u
        // needs only picks 0 .. u to know its expert.  Every wave routes the
        // token, requests its weights right after pick u and makes the
        // remaining picks while they stream, so the lower ranks' weights go
        // out before the whole top-k is known.
        l_load(0);
        RouteState rs;
        route_begin(rs, lg, E, lane);
        const int ur = min(u, k - 1);
        route_rounds(rs, 0, ur + 1, E, lane);
        e_rank = (int)readlane_u(rs.pick, ur);
        wait_vmem();   // the token's logits and activation rows are in
        issue_w13(e_rank);
        route_rounds(rs, ur + 1, k, E, lane);
        if (wave == 0) route_end(rs, k, ids_l, w_l, lane);
    } else {
        l_load(wave);
#pragma unroll 1
        for (int t = wave; t < M; t += 4) {
            if (t != wave) l_load(t);
            route_fast(lg, E, k, ids_l + t * k, w_l + t * k, lane);
        }
    }
    asm volatile("" : "+v"(epoch));   // the count is first needed here
    if (tid == 0) misc_l[3] = (int)(epoch + 1u);
    __syncthreads();
    if (wave == 0) {
        // experts 4l .. 4l + 3 of lane l present among the R <= 64 routes
        // (broadcast reads of the ids), then their ascending list by a prefix
        // sum
        int c[4] = {0, 0, 0, 0};
#pragma unroll 4
        for (int p = 0; p < R; ++p) {
            const int ep = ids_l[p];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] |= (ep == 4 * lane + j) ? 1 : 0;
        }        const int lact = c[0] + c[1] + c[2] + c[3];
        const int iact = wave_scan_incl(lact);
        int arun = iact - lact;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c[j]) act_l[arun++] = 4 * lane + j;
        if (lane == 63) misc_l[0] = iact;
    }
    __syncthreads();
    const int U = misc_l[0];
    const uint32_t tag = (uint32_t)misc_l[3];
    const bool has_unit = u < U;
    // the unit's expert: the u-th of the active experts in ascending order,
    // or for one token the u-th pick
    const int e = has_unit ? (MM == 1 ? e_rank : act_l[u]) : 0;

    // ---- the part's gate/up weights requested now (one token: already
    // requested during the routing, see phase 0)
    if constexpr (MM != 1) {
        // Nothing from phase 0 is still in flight; saying so keeps the
        // compiler from draining these loads at the waits below.
        wait_vmem();
        if (has_unit) issue_w13(e);
    }

    // ---- activation codes of every token into LDS (while the weights
    // stream): M * h / 128 <= 64 groups, one 16-lane row each
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int task = qbase + 16 * s4;
        if (task < nq) {
            const int t = task / G, g = task - t * G;
            const uint4 uu = xr[s4];
            float v[8] = {bf16_lo(uu.x), bf16_hi(uu.x), bf16_lo(uu.y), bf16_hi(uu.y),
                          bf16_lo(uu.z), bf16_hi(uu.z), bf16_lo(uu.w), bf16_hi(uu.w)};
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
            m = row16_max(m);
            const float sc = m / kE4M3Max;
            *reinterpret_cast<uint2*>(xq_l + t * h + g * 128 + col * 8) = quant8(v, sc);
            if (col == 0) xs_l[t * kFusedMaxKB + g] = sc;
        }
    }
    if (wave == 0) {
        // counts and each route's rank inside its expert (ballot match per
        // 64 routes), then offsets by a DPP prefix sum, then the routes in
        // (expert, route id) order
        for (int ee = lane; ee < E; ee += 64) cnt_l[ee] = 0;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int lr[4], ee4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            lr[b] = 0;
            ee4[b] = 0x1FF;
            if (64 * b < R) {
                const int p = 64 * b + lane;
                const int ep = p < R ? ids_l[p] : 0x1FF;
                const uint64_t same = match_id(ep);
                if (p < R) {
                    lr[b] = cnt_l[ep] + __popcll(same & below);
                    ee4[b] = ep;
                    if ((same >> lane) == 1ull) cnt_l[ep] += __popcll(same);
                }
            }
        }
        int c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = (4 * lane + j < E) ? cnt_l[4 * lane + j] : 0;
        const int lsum = c[0] + c[1] + c[2] + c[3];
        const int incl = wave_scan_incl(lsum);
        int run = incl - lsum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ej = 4 * lane + j;
            if (ej < E) off_l[ej] = run;
            run += c[j];
        }
        if (lane == 63) off_l[E] = incl;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int p = 64 * b + lane;
            if (p < R) srt_l[off_l[ee4[b]] + lr[b]] = p;
        }
        // the block scales (the first loads of the batch to arrive)
        if (has_unit) {
            if (lane >= 32 && lane < 48) sc2_l[lane - 32] = sc_v;
        }
    }
    __syncthreads();

    // The code below is straight-line wherever it touches memory: loads use
    // clamped (always valid) addresses and unused values are dropped by
    // selects, because a load under a lane-dependent condition makes the
    // compiler copy its result into place after a wait for it.
    const int beg = has_unit ? off_l[e] : 0;
    const int cnt = has_unit ? off_l[e + 1] - beg : 0;   // routes of expert e (<= M <= MM)
    const int cntc = cnt > 0 ? cnt : 1;
    const bool valid = col < cnt;
    const int pc = srt_l[beg + min(col, cntc - 1)];        // route of MFMA column col (clamped)
    const v8i zero = zero8();

    // ---- gate/up: raw MFMA block sums of this wave's K blocks into LDS
    if (has_unit) {
        const int tc = pc / k;
#pragma unroll
        for (int j = 0; j < kKBW; ++j) {
            const int kb = wave + 4 * j;
            if (kb < KB) {
                v8i B = load32(xq_l + tc * h + kb * 128 + kg * 32);
                B = valid ? B : zero;
#pragma unroll
                for (int t2 = 0; t2 < 2 * NT; ++t2) {
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f blk = mfma_16x16x128_e4m3(lines_to_frag(A[t2][j], bounce + (t2 & 1) * 2048, lane, col, kg),
                                                        B, z);
                    if (valid) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            blk_l[((t2 * 16 + 4 * kg + v) * MM + col) * kFusedMaxKB + kb] = blk[v];
                    }
                }
            }
        }
    }
    __syncthreads();
    // w2 (this wave's 16-row down tiles) is requested only now: the w13
    // requests of every workgroup go out first, so the gate/up inputs of the
    // whole layer arrive about a third of the stream earlier, and the w2
    // stream overlaps the exchange of the SiLU-mul values, which the down
    // MFMAs wait for anyway.  After the barrier, so that a wave held up
    // issuing them does not hold up wave 0's promotion.
    if (has_unit && wave >= kDW0) {
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            const int tt = min(wave - kDW0 + kDWN * j, ndt - 1);
            D[j] = load_lines_nt(a.w2 + ((size_t)e * h + q * drows + tt * 16) * i + ib * 128, i, lane);
        }
    }

    // ---- block promotion in K order: acc += blk * (s_act * s_w), the scale
    // product rounded first, then SiLU(gate) * up, published for the unit's
    // parts; one lane per (route, gate/up row pair)
    if (has_unit && wave == 0) {
#pragma unroll
        for (int rep = 0; rep < (MM * 16 * NT + 63) / 64; ++rep) {
#pragma clang fp contract(off)
            const int L = lane + 64 * rep;
            const int c = min(L / (16 * NT), cntc - 1), r = L % (16 * NT);
            const int tg = r >> 4, rr = r & 15;
            const int p = srt_l[beg + c];
            // this lane's 16 block sums of its gate row and of its up row, and
            // its token's 16 activation scales: 16-byte LDS reads (entries past
            // KB or G are dropped below); the weight scales come from lane kb
            // (gate) and lane 16 + kb (up) of wave 0 by readlane
            const float4* xsr = reinterpret_cast<const float4*>(xs_l + (p / k) * kFusedMaxKB);
            const float4* bgr = reinterpret_cast<const float4*>(blk_l + ((tg * 16 + rr) * MM + c) * kFusedMaxKB);
            const float4* bur = reinterpret_cast<const float4*>(blk_l + (((NT + tg) * 16 + rr) * MM + c) * kFusedMaxKB);
            float xv[kFusedMaxKB], bg[kFusedMaxKB], bu[kFusedMaxKB];
#pragma unroll
            for (int q4 = 0; q4 < kFusedMaxKB / 4; ++q4) {
                const float4 x4 = xsr[q4], g4 = bgr[q4], u4 = bur[q4];
                xv[4 * q4] = x4.x; xv[4 * q4 + 1] = x4.y; xv[4 * q4 + 2] = x4.z; xv[4 * q4 + 3] = x4.w;
                bg[4 * q4] = g4.x; bg[4 * q4 + 1] = g4.y; bg[4 * q4 + 2] = g4.z; bg[4 * q4 + 3] = g4.w;
                bu[4 * q4] = u4.x; bu[4 * q4 + 1] = u4.y; bu[4 * q4 + 2] = u4.z; bu[4 * q4 + 3] = u4.w;
            }
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int kb = 0; kb < kFusedMaxKB; ++kb) {
                const float swg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc_v), kb));
                const float swu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc_v), kFusedMaxKB + kb));
                const float tg_ = bg[kb] * (xv[kb] * swg);
                const float tu_ = bu[kb] * (xv[kb] * swu);
                ag = ag + (kb < KB ? tg_ : -0.0f);   // -0 added leaves any value unchanged
                au = au + (kb < KB ? tu_ : -0.0f);
            }
            const float v = (ag / (1.0f + expf(-ag))) * au;
            if (L < cnt * 16 * NT) st_agent64(a.v_ll + (size_t)p * i + ib * 128 + q * (128 / P) + r, ll_pack(v, tag));
        }

        // the unit's 128 SiLU-mul values of each route, from all its parts:
        // first the sentinel of every (route, part) -- the part's last column
        // -- then the values (lane l takes values 4(l % 32) .. +3; clamped
        // routes re-read a real one); amax, the scale amax/448 and the E4M3
        // codes into LDS
        const uint64_t* sent = nullptr;
        if (lane < cnt * P) {
            const int c = lane / P, qq = lane - c * P;
            sent = a.v_ll + (size_t)srt_l[beg + c] * i + ib * 128 + qq * (128 / P) + 128 / P - 1;
        }
        bool ok = wait_sentinel(sent, tag, err);
        const uint64_t* ptrs[4 * MM];
#pragma unroll
        for (int c = 0; c < MM; ++c) {
            const uint64_t* vp = a.v_ll + (size_t)srt_l[beg + min(c, cntc - 1)] * i + ib * 128 + 4 * (lane & 31);
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) ptrs[4 * c + m4] = vp + m4;
        }
        uint64_t w[4 * MM];
        ok = read_words<4 * MM>(ptrs, tag, w, err) && ok;
        const bool all_ok = __ballot(!ok) == 0ull;
#pragma unroll
        for (int c = 0; c < MM; ++c) {
            if (c < cnt) {
                float v4[4];
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) v4[m4] = ll_value(w[4 * c + m4]);
                float m = fmaxf(fmaxf(fabsf(v4[0]), fabsf(v4[1])), fmaxf(fabsf(v4[2]), fabsf(v4[3])));
                m = xor16_max(row16_max(m));   // lanes l and l + 32 hold the same values
                const float sc = all_ok ? m / kE4M3Max : __builtin_nanf("");
                const uint32_t codes = sc != 0.0f ? quant4(v4[0], v4[1], v4[2], v4[3], sc, __builtin_amdgcn_rcpf(sc)) : 0u;
                if (lane < 32) *reinterpret_cast<uint32_t*>(a2_l + c * 128 + 4 * lane) = codes;
                if (lane == 0) a2s_l[c] = sc;
            }
        }
    }
    // Waves that hold w2 tiles but have no exchange work (all but wave 0)
    // turn their tiles into MFMA fragments while wave 0 waits for the unit's
    // other parts, so that after the barrier only the MFMAs remain.
    const bool frag_early = wave > 0;
    if (has_unit && wave >= kDW0 && frag_early) {
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            const int tt = wave - kDW0 + kDWN * j;
            if (tt < ndt) D[j] = lines_to_frag(D[j], bounce + (j & 1) * 2048, lane, col, kg);
        }
    }
    __syncthreads();

    // ---- down: this part's rows times the unit's K block, published as block
    // terms blk * (a2s * s2) per route
    if (has_unit && wave >= kDW0) {
        const int cl = min(col, MM - 1);
        v8i B = load32(a2_l + cl * 128 + kg * 32);
        B = valid ? B : zero;
        const float a2sv = a2s_l[cl];
#pragma unroll
        for (int j = 0; j < NDT; ++j) {
            const int tt = wave - kDW0 + kDWN * j;
            if (tt < ndt) {
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v8i Af = frag_early ? D[j] : lines_to_frag(D[j], bounce + (j & 1) * 2048, lane, col, kg);
                const v4f blk = mfma_16x16x128_e4m3(Af, B, z);
                const int n0 = q * drows + tt * 16;
                const float sc = a2sv * sc2_l[n0 / 128 - nb0];
                if (valid) {
                    uint64_t* tp = a.t_ll + ((size_t)pc * IB + ib) * h + n0 + 4 * kg;
#pragma unroll
                    for (int v = 0; v < 4; ++v) st_agent64(tp + v, ll_pack(blk[v] * sc, tag));
                }
            }
        }
    }

    // ---- combine 64 output columns of a token: wave w sums the block terms
    // of ranks w, w + 4, ... over the blocks ascending, then wave 0 adds the
    // ranks in order with their routing weights
    const int nct = M * (h / 64);
    for (int ct = blockIdx.x; ct < nct; ct += gridDim.x) {
        const int t = ct / (h / 64), n = (ct - t * (h / 64)) * 64 + lane;
        // sentinels first: lane j < (ranks of this wave) * IB polls the last
        // column of this tile in the term row of (rank wave + 4 (j / IB),
        // block j % IB); then every rank and block slot reads a real word
        // (clamped duplicates of live words)
        const int nr = k > wave ? (k - wave + 3) / 4 : 0;   // ranks of this wave
        const uint64_t* sent = nullptr;
        if (lane < nr * IB) {
            const int rj = lane / IB, b = lane - rj * IB;
            sent = a.t_ll + ((size_t)(t * k + wave + 4 * rj) * IB + b) * h + (n - lane) + 63;
        }
        bool ok = wait_sentinel(sent, tag, err);
        const uint64_t* ptrs[4 * kFusedMaxIB];
#pragma unroll
        for (int rj = 0; rj < 4; ++rj) {
            const int r = min(wave + 4 * rj, k - 1);
#pragma unroll
            for (int b = 0; b < kFusedMaxIB; ++b)
                ptrs[rj * kFusedMaxIB + b] = a.t_ll + ((size_t)(t * k + r) * IB + min(b, IB - 1)) * h + n;
        }
        uint64_t w[4 * kFusedMaxIB];
        ok = read_words<4 * kFusedMaxIB>(ptrs, tag, w, err) && ok;
#pragma unroll
        for (int rj = 0; rj < 4; ++rj) {
#pragma clang fp contract(off)
            float y = 0.0f;
#pragma unroll
            for (int b = 0; b < kFusedMaxIB; ++b) y = y + (b < IB ? ll_value(w[rj * kFusedMaxIB + b]) : -0.0f);
            const int r = wave + 4 * rj;
            if (r < k) y_l[r * 64 + lane] = ok ? y : __builtin_nanf("");
        }
        __syncthreads();
        if (wave == 0) {
#pragma clang fp contract(off)
            float wv[16], yv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                wv[r] = w_l[min(t * k + r, R - 1)];
                yv[r] = y_l[r * 64 + lane];
            }
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float term = wv[r] * yv[r];
                acc = acc + (r < k ? term : -0.0f);
            }
            __bf16 bv = (__bf16)acc;
            a.out[(size_t)t * h + n] = __builtin_bit_cast(uint16_t, bv);
        }
        __syncthreads();
    }

    // Workgroup 0 publishes the batch's routing and quantisation (inspection).
    if (blockIdx.x == 0) {
        for (int p = tid; p < R; p += 256) {
            a.ids[p] = ids_l[p];
            a.tw[p] = w_l[p];
            a.sorted[p] = srt_l[p];
        }
        for (int ee = tid; ee < E; ee += 256) {
            a.offsets[ee] = off_l[ee];
            a.counts[ee] = off_l[ee + 1] - off_l[ee];
            a.active[ee] = ee < U ? act_l[ee] : 0;
        }
        if (tid == 0) {
            a.offsets[E] = off_l[E];
            *a.num_active = U;
        }
        for (int j = tid * 16; j < M * h; j += 256 * 16)
            *reinterpret_cast<uint4*>(a.xq + j) = *reinterpret_cast<const uint4*>(xq_l + j);
        for (int j = tid; j < M * G; j += 256) a.xs[j] = xs_l[(j / G) * kFusedMaxKB + j % G];
    }

    // ---- exit: the last workgroup advances the forward count
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomicAdd(a.sync + kSyncExit / 4, 1u);
        misc_l[4] = (old == gridDim.x - 1);
    }
    __syncthreads();
    if (misc_l[4]) {
        const uint32_t ep = tag - 1u;
        if (ep + 2u == 0u) {
            // the next tag would be 0, the value of a cleared word: clear the
            // exchange region and start counting again
            uint64_t* ll = a.v_ll;
            for (size_t j = tid; j < kLLBytes / 8; j += 256) st_agent64(ll + j, 0ull);
            wait_vmem();
            __syncthreads();
            if (tid == 0) st_agent(a.sync + kSyncEpoch / 4, 0u);
        } else if (tid == 0) {
            st_agent(a.sync + kSyncEpoch / 4, ep + 1u);
        }
        if (tid == 0) st_agent(a.sync + kSyncExit / 4, 0u);
    }
}

// Parts per unit for a batch: 8 when the grid of every possible unit fits,
// else 4, else 0 (not supported).
int fused_parts(int M, int i, int E, int k) {
    const int umax = std::min(E, M * k);
    const int units = umax * (i / 128);
    if (units * 8 <= kFusedMaxGrid) return 8;
    if (units * 4 <= kFusedMaxGrid) return 4;
    return 0;
}

template <int P>
static size_t lds_for(int M, int h, int E, int k) {
    switch (M) {
        case 1: return fused_lds<P, 1>(M, h, E, k).total;
        case 2: return fused_lds<P, 2>(M, h, E, k).total;
        case 3: return fused_lds<P, 3>(M, h, E, k).total;
        default: return fused_lds<P, 4>(M, h, E, k).total;
    }
}

size_t fused_lds_bytes(int M, int h, int i, int E, int k) {
    const int P = fused_parts(M, i, E, k);
    if (P == 8) return lds_for<8>(M, h, E, k);
    if (P == 4) return lds_for<4>(M, h, E, k);
    return 0;
}

bool fused_supported(int M, int h, int i, int E, int k) {
    const size_t R = (size_t)M * k, IB = (size_t)i / 128;
    return M >= 1 && M <= kFusedMaxM && k <= 16 && E <= 256 && h % 128 == 0 && h <= 128 * kFusedMaxKB &&
           (size_t)M * (h / 128) <= 64 &&
           i % 128 == 0 && IB <= kFusedMaxIB && fused_parts(M, i, E, k) > 0 &&
           fused_v_words(M, i, k) + R * IB * h <= kLLBytes / 8 && fused_lds_bytes(M, h, i, E, k) <= 64 * 1024;
}

// Launches one instance after checking that its whole grid can be resident
// at once (the workgroups wait on each other); the occupancy is queried once
// per device and LDS size.
template <int P, int MM>
static hipError_t launch_instance(const FusedArgs& args, int grid, size_t lds, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static int cached_cu[64] = {0};
    static size_t cached_lds[64] = {0};
    static int cached_blocks[64] = {0};
    if (cached_cu[dev] == 0 || cached_lds[dev] != lds) {
        int cu = 0, nb = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_decode_kernel<P, MM>, 256, lds) != hipSuccess)
            return hipErrorInvalidConfiguration;
        cached_cu[dev] = cu;
        cached_blocks[dev] = nb;
        cached_lds[dev] = lds;
    }
    if (cached_cu[dev] * cached_blocks[dev] < grid) return hipErrorInvalidConfiguration;
    launch((fused_decode_kernel<P, MM>), dim3(grid), dim3(256), lds, stream, args);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_parts(const FusedArgs& args, int grid, size_t lds, hipStream_t stream) {
    switch (args.M) {
        case 1: return launch_instance<P, 1>(args, grid, lds, stream);
        case 2: return launch_instance<P, 2>(args, grid, lds, stream);
        case 3: return launch_instance<P, 3>(args, grid, lds, stream);
        case 4: return launch_instance<P, 4>(args, grid, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused_decode(const FusedArgs& args, hipStream_t stream) {
    const int P = fused_parts(args.M, args.i, args.E, args.k);
    const size_t lds = fused_lds_bytes(args.M, args.h, args.i, args.E, args.k);
    const int grid = std::min(args.E, args.M * args.k) * (args.i / 128) * P;
    if (P == 8) return launch_parts<8>(args, grid, lds, stream);
    if (P == 4) return launch_parts<4>(args, grid, lds, stream);
    return hipErrorInvalidValue;
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n; j += (size_t)gridDim.x * 256)
        p[j] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, size_t words, hipStream_t stream) {
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, stream, p, words);
    return hipGetLastError();
}

}  // namespace moe
