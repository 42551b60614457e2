// fused_decode.hip -- the whole layer in one persistent kernel for small
// batches (M <= 16 tokens): decode and speculative verification.
//
// Every workgroup first recomputes, on chip, what it needs from the batch:
// the router top-k of all M tokens (one wave per token: DPP row maxima,
// scalar readlanes and ballots; the picked logits come back out of the keys),
// the 1x128 E4M3 activation codes of all tokens (into LDS) and the grouping
// of the M*k routes by expert (ballot ranks, DPP prefix sums).  Work is then
// split in two task lists:
//
//  A task (expert slot u, 128-column group jg, quarter q): 32 gate rows and
//    the matching 32 up rows of w13[e_u], K = h, streamed once with
//    v_mfma_f32_16x16x128_f8f6f4 (weights as A, the expert's <= 16 routes as
//    B), per-128-K-block scale promotion; FP32 results per route (Netra
//    compiler architecture page: gate/up FP32).
//  B task (expert slot u, 64-row tile of w2[e_u]): its weights are loaded
//    into registers before the workgroup's gate/up work is computed; it then
//    computes SiLU(gate) * up of u's routes and their 1x128 E4M3
//    requantisation straight into LDS (Netra Kernel README, MoE prefill pair:
//    SiLU and quantisation), and the fp32 partial rows (down-partial).
//  Combine: the workgroup that owns a token's last-rank route for a tile
//    sums that tile's k partials in rank order and writes bf16 (route
//    reducer; Inferact amd-kernels README, atomics rule: no atomic sums, a
//    fixed order).  It does so only after all of its own B tasks.
//
// Exchange between workgroups: each gate/up result and each partial is one
// 64-bit word (value, tag of this forward) written and read with
// agent-coherent stores and loads; a consumer polls the words it needs until
// they carry this forward's tag.  The data is its own flag, so there are no
// counters to contend on and no cache-wide fences.  The tag is the
// workspace's forward count plus one, read at the start; the last workgroup
// to exit advances it (and, once every 2^32 forwards, clears the exchange
// region so that no stale word can ever carry a current tag).  Waits are
// bounded in time; a timeout sets a sticky error word instead of hanging.
// Tasks only wait on tasks of an earlier phase, and the grid never exceeds
// the number of workgroups that can be resident at once, so every awaited
// task is always running.
#include "device.h"
#include "fused_decode.h"

namespace moe {

constexpr int kFusedMaxM = 16;
constexpr int kFusedMaxIB = 8;              // i <= 1024
constexpr int kMaxKB = 16;                  // gate/up K blocks loaded per batch
constexpr int kQuarters = 4;                // A task: 32 gate + 32 up rows
constexpr int kDownRows = 64;               // B task rows
constexpr uint64_t kWaitTicks = 100000000;  // 1 s of the 100 MHz constant clock

__device__ __forceinline__ uint32_t readlane_u(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Router of one token on one wave; lane l holds the logits of experts
// l + 64j.  Each pick: a DPP max over each 16-lane row, the four row maxima
// read into scalars, and the lowest expert index holding that key found by
// ballot (ties go to the lower index, -0 equals +0).  Lane r keeps pick r;
// the weights exp(l_r - l_0) / sum are summed in rank order.
__device__ __forceinline__ void route_fast(const float lg[4], int E, int k, int* ids_l,
                                           float* w_l, int lane) {
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = (lane + 64 * j < E) ? float_order_key(lg[j]) : 0u;
    int my_pick = 0;
    float my_l = 0.0f, l0 = 0.0f;
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        uint32_t m = max(max(key[0], key[1]), max(key[2], key[3]));
        m = row16_max_u(m);
        const uint32_t smax = max(max(readlane_u(m, 0), readlane_u(m, 16)),
                                  max(readlane_u(m, 32), readlane_u(m, 48)));
        int e = E - 1;   // only reached for NaN logits (outside the contract)
        if (smax != 0u) {
            const uint64_t b0 = __ballot(key[0] == smax);
            const uint64_t b1 = __ballot(key[1] == smax);
            const uint64_t b2 = __ballot(key[2] == smax);
            const uint64_t b3 = __ballot(key[3] == smax);
            e = b0 ? __builtin_ctzll(b0)
              : b1 ? 64 + __builtin_ctzll(b1)
              : b2 ? 128 + __builtin_ctzll(b2)
              : b3 ? 192 + __builtin_ctzll(b3) : E - 1;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane + 64 * j == e) key[j] = 0u;
        const float lv = float_from_order_key(smax);
        if (r == 0) l0 = lv;
        if (lane == r) {
            my_pick = e;
            my_l = lv;
        }
    }
    const float ex = lane < k ? expf(my_l - l0) : 0.0f;
    float sum = 0.0f;
#pragma unroll 1
    for (int r = 0; r < k; ++r) sum += __uint_as_float(readlane_u(__float_as_uint(ex), r));
    if (lane < k) {
        ids_l[lane] = my_pick;
        w_l[lane] = ex / sum;
    }
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

// SiLU(gate) * up of one 128-column group of one route on one 16-lane row,
// requantised to E4M3 into LDS.  The lane's 16 gate/up words are loaded
// together and reloaded together until they all carry this forward's tag.
__device__ __forceinline__ void silu_quant_ll(const uint64_t* __restrict__ gate,
                                              const uint64_t* __restrict__ up, int sub,
                                              uint32_t tag, uint32_t* err, uint8_t* q, float* s) {
    uint64_t wg[8], wu[8];
    uint64_t t0 = 0;
    for (int tries = 0;; ++tries) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            wg[j] = ld_agent64(gate + sub * 8 + j);
            wu[j] = ld_agent64(up + sub * 8 + j);
        }
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 8; ++j) ok = ok && ll_tag(wg[j]) == tag && ll_tag(wu[j]) == tag;
        if (ok) break;
        if (tries == 0) t0 = wall_clock64();
        if (wall_clock64() - t0 > kWaitTicks) {
            atomicOr(err, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    float v[8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float a = ll_value(wg[j]);
        v[j] = (a / (1.0f + expf(-a))) * ll_value(wu[j]);
        m = fmaxf(m, fabsf(v[j]));
    }
    m = row16_max(m);
    const float sc = m / kE4M3Max;
    *reinterpret_cast<uint2*>(q + sub * 8) = quant8(v, sc);
    if (sub == 0) *s = sc;
}

__global__ __launch_bounds__(256) void fused_decode_kernel(FusedArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int M = a.M, h = a.h, i = a.i, E = a.E, k = a.k;
    const int R = M * k, G = h / 128, IB = i / 128, KB = h / 128, N13 = 2 * i;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    uint32_t* err = a.sync + kSyncErr / 4;

    // ---- LDS carve (all offsets 16-byte aligned)
    uint8_t* xq_l = smem;                                            // [M][h]
    float* xs_l = reinterpret_cast<float*>(xq_l + M * h);            // [M][G]
    int* ids_l = reinterpret_cast<int*>(xs_l + ((M * G + 3) & ~3));  // [R]
    float* w_l = reinterpret_cast<float*>(ids_l + ((R + 3) & ~3));   // [R]
    int* off_l = reinterpret_cast<int*>(w_l + ((R + 3) & ~3));       // [E+1]
    int* act_l = off_l + ((E + 1 + 3) & ~3);                         // [E]
    int* srt_l = act_l + ((E + 3) & ~3);                             // [R]
    int* cnt_l = srt_l + ((R + 3) & ~3);                             // [E]
    int* misc_l = cnt_l + ((E + 3) & ~3);                            // [32]
    uint8_t* a2_l = reinterpret_cast<uint8_t*>(misc_l + 32);         // [16][i + 16]
    const int a2_stride = i + 16;
    float* a2s_l = reinterpret_cast<float*>(a2_l + 16 * a2_stride);  // [16][IB]

    // ---- phase 0: tag, routing, activation codes and grouping.  The first
    // token's logits and the first batch of x rows are requested before any
    // of them is used.
    // The forward count is read now and stored to LDS only after routing, so
    // that its load does not hold up the logits and x loads behind it.
    uint32_t epoch = 0u;
    if (tid == 0) epoch = ld_agent(a.sync + kSyncEpoch / 4);
    uint32_t* bm_l = reinterpret_cast<uint32_t*>(misc_l + 8);   // experts present in the batch
    if (tid < 8) bm_l[tid] = 0u;
    const int nq = M * G;   // 16-lane rows of activation groups
    const int qbase = wave * 4 + (lane >> 4);
    uint4 xr[4];
    auto x_load = [&](int base) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int task = base + 16 * s4;
            if (task < nq) {
                const int t = task / G, g = task - t * G;
                xr[s4] = *reinterpret_cast<const uint4*>(a.x + (size_t)t * h + g * 128 + col * 8);
            }
        }
    };
    float lg[4];
    auto l_load = [&](int t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            lg[j] = (t < M && e < E) ? a.logits[(size_t)t * E + e] : 0.0f;
        }
    };
    l_load(wave);
    x_load(qbase);
#pragma unroll 1
    for (int t = wave; t < M; t += 4) {
        if (t != wave) l_load(t);
        route_fast(lg, E, k, ids_l + t * k, w_l + t * k, lane);
    }
    asm volatile("" : "+v"(epoch));   // the count is first needed here
    if (tid == 0) misc_l[3] = (int)(epoch + 1u);
    // the active experts (ascending) right after routing, so that the weight
    // prefetch below is in flight while the activations are quantised and
    // the routes grouped
    __syncthreads();
    for (int p = tid; p < R; p += 256) atomicOr(&bm_l[ids_l[p] >> 5], 1u << (ids_l[p] & 31));
    __syncthreads();
    if (wave == 0) {
        int c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            c[j] = e < E ? (int)((bm_l[e >> 5] >> (e & 31)) & 1u) : 0;
        }
        const int lact = c[0] + c[1] + c[2] + c[3];
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
    const int nA = U * IB * kQuarters;
    const int NT = h / kDownRows;
    const int nB = U * NT;

    // ---- prefetch: the first gate/up task's first K batch (or, without gate/up
    // work, the first down task's weights)
    // weights in registers; each task's 16 (8) block scales arrive as one
    // lane-indexed load (lane j holds block j's scale) and are read back with
    // readlane
    v8i Aw[kMaxKB];
    float Asc_v = 0.0f;
    v8i Bw[kFusedMaxIB];
    float Bsc_v = 0.0f;
    auto a_geom = [&](int task, int& u, int& e, int& row0) {
        u = task / (IB * kQuarters);
        const int rem = task - u * IB * kQuarters;
        const int jg = rem / kQuarters, q = rem - jg * kQuarters;
        e = act_l[u];
        row0 = (wave >> 1) * i + jg * 128 + q * 32 + (wave & 1) * 16;
    };
    auto a_load = [&](int e, int row0, int kb0) {
        const uint8_t* wrow = a.w13 + ((size_t)e * N13 + row0 + col) * h + kg * 32 + kb0 * 128;
        const float* ws = a.s13 + ((size_t)e * (N13 / 128) + row0 / 128) * KB + kb0;
        const int nkb = min(KB - kb0, kMaxKB);
        if (lane < nkb) Asc_v = ws[lane];
#pragma unroll
        for (int u8 = 0; u8 < kMaxKB; ++u8)
            if (u8 < nkb) Aw[u8] = load32(wrow + u8 * 128);
    };
    auto b_load = [&](int task) {
        const int u = task / NT, nt = task - u * NT;
        const int e = act_l[u];
        const int n0 = nt * kDownRows + wave * 16;
        const uint8_t* wrow = a.w2 + ((size_t)e * h + n0 + col) * i + kg * 32;
        const float* ws = a.s2 + ((size_t)e * (h / 128) + n0 / 128) * IB;
        if (lane < IB) Bsc_v = ws[lane];
#pragma unroll
        for (int kb = 0; kb < kFusedMaxIB; ++kb)
            if (kb < IB) Bw[kb] = load32(wrow + kb * 128);
    };
    // nothing from phase 0 is still in flight (its loads were consumed);
    // saying so keeps the compiler from draining the prefetch below later on
    wait_vmem();
    if ((int)blockIdx.x < nA) {
        int u, e, row0;
        a_geom(blockIdx.x, u, e, row0);
        a_load(e, row0, 0);
    } else if ((int)blockIdx.x < nB) {
        b_load(blockIdx.x);   // no gate/up work here: fetch the down tile now
    }

#pragma unroll 1
    for (int base = qbase; base < nq; base += 64) {
        if (base != qbase) x_load(base);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int task = base + 16 * s4;
            if (task < nq) {
                const int t = task / G, g = task - t * G;
                const uint4 u = xr[s4];
                float v[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                              bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
                m = row16_max(m);
                const float sc = m / kE4M3Max;
                *reinterpret_cast<uint2*>(xq_l + t * h + g * 128 + col * 8) = quant8(v, sc);
                if (col == 0) xs_l[t * G + g] = sc;
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        // counts and each route's rank inside its expert (ballot match per
        // 64 routes), then offsets by a DPP prefix sum, then the routes in
        // (expert, route id) order
        for (int e = lane; e < E; e += 64) cnt_l[e] = 0;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int lr[4], ee[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            lr[b] = 0;
            ee[b] = 0x1FF;
            if (64 * b < R) {
                const int p = 64 * b + lane;
                const int e = p < R ? ids_l[p] : 0x1FF;
                const uint64_t same = match_id(e);
                if (p < R) {
                    lr[b] = cnt_l[e] + __popcll(same & below);
                    ee[b] = e;
                    if ((same >> lane) == 1ull) cnt_l[e] += __popcll(same);
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
            const int e = 4 * lane + j;
            if (e < E) off_l[e] = run;
            run += c[j];
        }
        if (lane == 63) off_l[E] = incl;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int p = 64 * b + lane;
            if (p < R) srt_l[off_l[ee[b]] + lr[b]] = p;
        }
    }
    __syncthreads();

    // ---- phase 1: gate/up quarters
    for (int task = blockIdx.x; task < nA; task += gridDim.x) {
        int u, e, row0;
        a_geom(task, u, e, row0);
        const int beg = off_l[e], cnt = off_l[e + 1] - beg;
        const bool valid = col < cnt;
        const int p = valid ? srt_l[beg + col] : 0;
        const int t = p / k;
        const uint8_t* xrow = xq_l + t * h + kg * 32;
        const float* xsr = xs_l + t * G;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb0 = 0; kb0 < KB; kb0 += kMaxKB) {
            if (kb0 > 0 || task != (int)blockIdx.x) a_load(e, row0, kb0);
#pragma unroll
            for (int u8 = 0; u8 < kMaxKB; ++u8) {
                const int kb = kb0 + u8;
                if (kb < KB) {
                    const v8i B = valid ? load32(xrow + kb * 128) : zero8();
                    const float sc = (valid ? xsr[kb] : 0.0f) * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Asc_v), u8));
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f blk = mfma_16x16x128_e4m3(Aw[u8], B, z);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
                }
            }
        }
        if (valid) {
            uint64_t* gp = a.g_ll + (size_t)p * N13 + row0 + kg * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) st_agent64(gp + v, ll_pack(acc[v], tag));
        }
    }

    // The down tile's weights are fetched only now by workgroups that had
    // gate/up work: they are not needed before the gate/up results of the
    // whole route are in, and fetching them earlier only competes with the
    // gate/up weights for bandwidth.
    if ((int)blockIdx.x < nA && (int)blockIdx.x < nB) b_load(blockIdx.x);

    // ---- phase 2: down tiles
    for (int task = blockIdx.x; task < nB; task += gridDim.x) {
        const int u = task / NT, nt = task - u * NT;
        const int e = act_l[u];
        const int beg = off_l[e], cnt = off_l[e + 1] - beg;
        const int n0 = nt * kDownRows + wave * 16;
        if (task != (int)blockIdx.x) b_load(task);
#pragma unroll 1
        for (int r2 = wave * 4 + (lane >> 4); r2 < cnt * IB; r2 += 16) {
            const int jr = r2 / IB, b = r2 - jr * IB;
            const uint64_t* gr = a.g_ll + (size_t)srt_l[beg + jr] * N13 + b * 128;
            silu_quant_ll(gr, gr + i, col, tag, err, a2_l + jr * a2_stride + b * 128,
                          a2s_l + jr * IB + b);
        }
        __syncthreads();
        const bool valid = col < cnt;
        const int p = valid ? srt_l[beg + col] : 0;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < kFusedMaxIB; ++kb) {
            if (kb < IB) {
                const v8i B = valid ? load32(a2_l + col * a2_stride + kb * 128 + kg * 32) : zero8();
                const float sc = (valid ? a2s_l[col * IB + kb] : 0.0f) *
                                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Bsc_v), kb));
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f blk = mfma_16x16x128_e4m3(Bw[kb], B, z);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
            }
        }
        if (valid) {
            uint64_t* yp = a.y_ll + (size_t)p * h + n0 + kg * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) st_agent64(yp + v, ll_pack(acc[v], tag));
        }
        __syncthreads();
    }

    // ---- phase 3: combine the tiles of the tokens whose last-rank route this
    // workgroup computed (after all of its own down tiles)
    for (int task = blockIdx.x; task < nB; task += gridDim.x) {
        const int u = task / NT, nt = task - u * NT;
        const int e = act_l[u];
        const int beg = off_l[e], cnt = off_l[e + 1] - beg;
        for (int jr = 0; jr < cnt; ++jr) {
            const int pr = srt_l[beg + jr];
            if (pr % k != k - 1) continue;
            const int t = pr / k;
            if (tid < kDownRows) {
#pragma clang fp contract(off)
                // the k partials of column n, loaded together until all are
                // from this forward, then summed in rank order
                const int n = nt * kDownRows + tid;
                const uint64_t* yc = a.y_ll + (size_t)t * k * h + n;
                uint64_t w[16];
                uint64_t t0 = 0;
                for (int tries = 0;; ++tries) {
                    bool ok = true;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if (r < k) {
                            w[r] = ld_agent64(yc + (size_t)r * h);
                            ok = ok && ll_tag(w[r]) == tag;
                        }
                    }
                    if (ok) break;
                    if (tries == 0) t0 = wall_clock64();
                    if (wall_clock64() - t0 > kWaitTicks) {
                        atomicOr(err, 1u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                float accum = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (r < k) accum = accum + w_l[t * k + r] * ll_value(w[r]);
                __bf16 bv = (__bf16)accum;
                a.out[(size_t)t * h + n] = __builtin_bit_cast(uint16_t, bv);
            }
        }
    }

    // Workgroup 0 publishes the batch's routing and quantisation (inspection).
    if (blockIdx.x == 0) {
        for (int p = tid; p < R; p += 256) {
            a.ids[p] = ids_l[p];
            a.tw[p] = w_l[p];
            a.sorted[p] = srt_l[p];
        }
        for (int e = tid; e < E; e += 256) {
            a.offsets[e] = off_l[e];
            a.counts[e] = off_l[e + 1] - off_l[e];
            a.active[e] = e < U ? act_l[e] : 0;
        }
        if (tid == 0) {
            a.offsets[E] = off_l[E];
            *a.num_active = U;
        }
        for (int j = tid * 16; j < M * h; j += 256 * 16)
            *reinterpret_cast<uint4*>(a.xq + j) = *reinterpret_cast<const uint4*>(xq_l + j);
        for (int j = tid; j < M * G; j += 256) a.xs[j] = xs_l[j];
    }

    // ---- exit: the last workgroup advances the forward count
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomicAdd(a.sync + kSyncExit / 4, 1u);
        misc_l[4] = (old == gridDim.x - 1);
    }
    __syncthreads();
    if (misc_l[4]) {
        const uint32_t epoch = tag - 1u;
        if (epoch + 2u == 0u) {
            // the next tag would be 0, the value of a cleared word: clear the
            // exchange region and start counting again
            uint64_t* ll = a.g_ll;
            for (size_t j = tid; j < kLLBytes / 8; j += 256) st_agent64(ll + j, 0ull);
            wait_vmem();
            __syncthreads();
            if (tid == 0) st_agent(a.sync + kSyncEpoch / 4, 0u);
        } else if (tid == 0) {
            st_agent(a.sync + kSyncEpoch / 4, epoch + 1u);
        }
        if (tid == 0) st_agent(a.sync + kSyncExit / 4, 0u);
    }
}

size_t fused_lds_bytes(int M, int h, int i, int E, int k) {
    const int R = M * k, G = h / 128;
    auto r4 = [](int v) { return (size_t)((v + 3) & ~3); };
    size_t b = (size_t)M * h;
    b += r4(M * G) * 4;
    b += r4(R) * 4 * 2;
    b += r4(E + 1) * 4 + r4(E) * 4 + r4(R) * 4 + r4(E) * 4 + 32 * 4;
    b += (size_t)16 * (i + 16) + ((size_t)16 * kFusedMaxIB + 64) * 4;   // a2, a2 scales, router scratch
    return (b + 15) & ~(size_t)15;
}

bool fused_supported(int M, int h, int i, int E, int k) {
    const size_t R = (size_t)M * k, words = kLLBytes / 16;   // each exchange buffer: 4 MiB
    return M >= 1 && M <= kFusedMaxM && k <= 16 && E <= 256 && h % 128 == 0 && i % 128 == 0 &&
           i / 128 <= kFusedMaxIB && (size_t)M * h <= 32768 && h % kDownRows == 0 &&
           R * 2 * i <= words && R * h <= words && fused_lds_bytes(M, h, i, E, k) <= 64 * 1024;
}

// Workgroups that can be resident at once, per device (queried once).
static int resident_capacity(size_t lds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static int cached_cu[64] = {0};
    static size_t cached_lds[64] = {0};
    static int cached_blocks[64] = {0};
    if (dev < 0 || dev >= 64) return 0;
    if (cached_cu[dev] == 0 || cached_lds[dev] != lds) {
        int cu = 0, nb = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_decode_kernel, 256, lds) !=
            hipSuccess)
            return 0;
        cached_cu[dev] = cu;
        cached_blocks[dev] = nb;
        cached_lds[dev] = lds;
    }
    return cached_cu[dev] * cached_blocks[dev];
}

hipError_t launch_fused_decode(const FusedArgs& args, hipStream_t stream) {
    const size_t lds = fused_lds_bytes(args.M, args.h, args.i, args.E, args.k);
    const int cap = resident_capacity(lds);
    if (cap <= 0) return hipErrorInvalidConfiguration;
    const int IB = args.i / 128;
    const int umax = std::min(args.E, args.M * args.k);
    const int want = std::max(umax * IB * kQuarters, umax * (args.h / kDownRows));
    const int grid = std::max(1, std::min(cap, want));
    hipLaunchKernelGGL(fused_decode_kernel, dim3(grid), dim3(256), lds, stream, args);
    return hipGetLastError();
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
