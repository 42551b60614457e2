// route_quant.h -- the router top-k and the 1x128 activation quantiser as
// wave-level device functions, shared by the routing launches and the
// prefill producer (the algorithm is described in route_quant.hip).
#pragma once

#include "device.h"

namespace moe {

// Unsigned min over the 16 lanes of each DPP row.
__device__ __forceinline__ uint32_t row16_min_u(uint32_t v) {
    v = min(v, dpp_u<kDppQuadXor1>(v));
    v = min(v, dpp_u<kDppQuadXor2>(v));
    v = min(v, dpp_u<kDppRowHalfMirror>(v));
    v = min(v, dpp_u<kDppRowMirror>(v));
    return v;
}

// Unsigned max / min over the whole wave (DPP inside each row of 16, then
// the two row swaps); every lane gets the result.
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

// A lane's router candidates: keys (order-preserving bits of the logits, 0 =
// none) and their experts.  Bitonic network into pick order: key descending,
// expert ascending on equal keys.
template <int NQ>
__device__ __forceinline__ void sort_candidates(uint32_t (&key)[NQ], uint32_t (&idx)[NQ]) {
#pragma unroll
    for (int kk = 2; kk <= NQ; kk *= 2) {
#pragma unroll
        for (int jj = kk / 2; jj > 0; jj /= 2) {
#pragma unroll
            for (int a = 0; a < NQ; ++a) {
                const int b = a ^ jj;
                if (b > a) {
                    // ((a & kk) == 0): slot a takes the element that comes first
                    const bool b_first = key[b] > key[a] || (key[b] == key[a] && idx[b] < idx[a]);
                    const bool swap = ((a & kk) == 0) == b_first;
                    const uint32_t ka = key[a], ia = idx[a];
                    key[a] = swap ? key[b] : ka;
                    idx[a] = swap ? idx[b] : ia;
                    key[b] = swap ? ka : key[b];
                    idx[b] = swap ? ia : idx[b];
                }
            }
        }
    }
}

// The lane whose head is expert e drops it.  The pop is a bit mask the
// compiler cannot see through: as a condition the shift became a
// register-indexed select chain.
template <int NQ>
__device__ __forceinline__ void pop_candidate(uint32_t (&key)[NQ], uint32_t (&idx)[NQ], int e) {
    uint32_t pm = ((int)idx[0] == e && key[0] != 0u) ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(pm));
#pragma unroll
    for (int q = 0; q + 1 < NQ; ++q) {
        key[q] = (key[q + 1] & pm) | (key[q] & ~pm);
        idx[q] = (idx[q + 1] & pm) | (idx[q] & ~pm);
    }
    key[NQ - 1] &= ~pm;
}

// Router of one token on one wave: lane l holds the logits of experts
// l + 64 q, sorted once per lane (key descending, expert ascending).  A pick
// is the wave maximum of the lanes' head keys, then the lowest expert among
// the heads that reach it; the winning lane pops its head.  Equal logits go
// to the lower expert index and -0 equals +0.  Each pick's exp(l - l_0) is
// added to the rank-order sum as it comes; lane r stores pick r.
// coherent: store the ids with device-coherent stores (read by another
// workgroup of the same launch).
template <int NQ>
__device__ __forceinline__ void router_wave_nq(const float* __restrict__ l, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w,
                                               int lane, bool coherent) {
    // Unconditional loads (an index past E reads expert E - 1 and its key is
    // dropped), issued together.
    float lv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) lv[q] = l[min(lane + 64 * q, E - 1)];
    uint32_t key[NQ], idx[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        idx[q] = (uint32_t)(lane + 64 * q);
        key[q] = (int)idx[q] < E ? float_order_key(lv[q]) : 0u;
    }
    sort_candidates<NQ>(key, idx);
    int my_e = 0;
    float lmax = 0.0f, sum = 0.0f, my_ex = 0.0f;
    for (int rr = 0; rr < k; ++rr) {
        const uint32_t m = wave_max_u(key[0]);
        int e = (int)wave_min_u(key[0] == m ? idx[0] : 0xFFFFu);
        e = (m == 0u || e >= E) ? E - 1 : e;   // only for NaN logits (outside the contract)
        pop_candidate<NQ>(key, idx, e);
        const float pv = float_from_order_key(m);   // the pick's logit (-0 comes back as +0)
        if (rr == 0) lmax = pv;
        const float ex = expf(pv - lmax);
        sum += ex;
        if (lane == rr) {
            my_e = e;
            my_ex = ex;
        }
    }
    if (lane < k) {
        if (coherent) st_agent(reinterpret_cast<uint32_t*>(ids) + lane, (uint32_t)my_e);
        else ids[lane] = my_e;
        w[lane] = my_ex / sum;
    }
}

__device__ __forceinline__ void router_wave(const float* __restrict__ l, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int lane, bool coherent = false) {
    if (E <= 64)
        router_wave_nq<1>(l, E, k, ids, w, lane, coherent);
    else if (E <= 128)
        router_wave_nq<2>(l, E, k, ids, w, lane, coherent);
    else
        router_wave_nq<4>(l, E, k, ids, w, lane, coherent);
}

// Each 16-lane row of a wave takes one 128-wide group per step; the loads of
// kQuantBatch steps (from step st0) are issued before any group is processed.
constexpr int kQuantBatch = 4;
__device__ __forceinline__ int act_quant_steps(int K, int nwaves) { return (K / 128 + 4 * nwaves - 1) / (4 * nwaves); }

__device__ __forceinline__ void act_quant_load(const uint16_t* __restrict__ x, int K, int st0, int wave, int nwaves,
                                               int lane, uint4 u[kQuantBatch]) {
    const int G = K / 128, steps = act_quant_steps(K, nwaves), sub = lane & 15;
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        const int g = ((st0 + j) * nwaves + wave) * 4 + (lane >> 4);
        u[j] = make_uint4(0u, 0u, 0u, 0u);
        if (st0 + j < steps && g < G) u[j] = *reinterpret_cast<const uint4*>(x + g * 128 + sub * 8);
    }
}

// kCoh: codes and scales go out with device-scope stores (read by other
// workgroups of the same launch).
template <bool kCoh = false>
__device__ __forceinline__ void act_quant_process(int K, uint8_t* __restrict__ q, float* __restrict__ s, int st0,
                                                  int wave, int nwaves, int lane, const uint4 u[kQuantBatch]) {
    const int G = K / 128, steps = act_quant_steps(K, nwaves), sub = lane & 15;
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        if (st0 + j >= steps) break;
        const int g = ((st0 + j) * nwaves + wave) * 4 + (lane >> 4);
        float v[8] = {bf16_lo(u[j].x), bf16_hi(u[j].x), bf16_lo(u[j].y), bf16_hi(u[j].y),
                      bf16_lo(u[j].z), bf16_hi(u[j].z), bf16_lo(u[j].w), bf16_hi(u[j].w)};
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) a = fmaxf(a, fabsf(v[c]));
        a = row16_max(a);
        const float sc = a / kE4M3Max;
        if (g < G) {
            const uint2 c = quant8(v, sc);
            if constexpr (kCoh) {
                st_agent64(reinterpret_cast<uint64_t*>(q + g * 128 + sub * 8), (uint64_t)c.x | ((uint64_t)c.y << 32));
                if (sub == 0) st_agent(s + g, sc);
            } else {
                *reinterpret_cast<uint2*>(q + g * 128 + sub * 8) = c;
                if (sub == 0) s[g] = sc;
            }
        }
    }
}

// Quantise the rest of a row whose first kQuantBatch steps' loads are in u.
template <bool kCoh = false>
__device__ __forceinline__ void act_quant_finish(const uint16_t* __restrict__ x, int K, uint8_t* __restrict__ q,
                                                 float* __restrict__ s, int wave, int nwaves, int lane,
                                                 uint4 u[kQuantBatch]) {
    const int steps = act_quant_steps(K, nwaves);
    act_quant_process<kCoh>(K, q, s, 0, wave, nwaves, lane, u);
    for (int st0 = kQuantBatch; st0 < steps; st0 += kQuantBatch) {
        act_quant_load(x, K, st0, wave, nwaves, lane, u);
        act_quant_process<kCoh>(K, q, s, st0, wave, nwaves, lane, u);
    }
}

template <bool kCoh = false>
__device__ __forceinline__ void act_quant_row(const uint16_t* __restrict__ x, int K,
                                              uint8_t* __restrict__ q, float* __restrict__ s,
                                              int wave, int nwaves, int lane) {
    uint4 u[kQuantBatch];
    act_quant_load(x, K, 0, wave, nwaves, lane, u);
    act_quant_finish<kCoh>(x, K, q, s, wave, nwaves, lane, u);
}

// Router of four tokens on one wave: DPP row r (16 lanes) routes token
// t0 + r, lane j of a row holding the logits of experts j, j + 16, ...  Each
// lane first sorts its NQ candidates once (bitonic network on (key
// descending, expert ascending), key = order-preserving bits of the logit),
// so a round only looks at the lanes' heads: the row maximum of the head
// keys, then the lowest expert among the heads that reach it (four DPP steps
// each, inside the row), and the winning lane pops its head.  Equal logits go
// to the lower expert index and -0 equals +0.  The pick's logit is the same
// in every lane of the row, so each round adds its exponential to the
// rank-order sum right away; lane j keeps pick j.
template <int NQ>
__device__ __forceinline__ void router_rows16_nq(const float* __restrict__ logits, int t0, int M, int E, int k,
                                                 int32_t* __restrict__ ids, float* __restrict__ w, int lane) {
    const int r = lane >> 4, j = lane & 15, t = t0 + r;
    const bool live = t < M;
    const float* l = logits + (size_t)(live ? t : t0) * E;
    // Unconditional loads (an index past E reads expert E - 1 and its key is
    // dropped): under a per-lane condition each load was waited for before
    // the next was issued.
    float lv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) lv[q] = l[min(j + 16 * q, E - 1)];
    uint32_t key[NQ], idx[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        idx[q] = (uint32_t)(j + 16 * q);
        key[q] = (int)idx[q] < E ? float_order_key(lv[q]) : 0u;
    }
    sort_candidates<NQ>(key, idx);
    int my_e = 0;
    float lmax = 0.0f, sum = 0.0f, my_ex = 0.0f;
    for (int rr = 0; rr < k; ++rr) {
        const uint32_t m = row16_max_u(key[0]);
        int e = (int)row16_min_u(key[0] == m ? idx[0] : 0xFFFFu);
        e = (m == 0u || e >= E) ? E - 1 : e;   // only for NaN logits (outside the contract)
        pop_candidate<NQ>(key, idx, e);
        const float pv = float_from_order_key(m);
        if (rr == 0) lmax = pv;
        const float ex = expf(pv - lmax);
        sum += ex;
        if (j == rr) {
            my_e = e;
            my_ex = ex;
        }
    }
    if (live && j < k) {
        ids[(size_t)t * k + j] = my_e;
        w[(size_t)t * k + j] = my_ex / sum;
    }
}

__device__ __forceinline__ void router_rows16(const float* __restrict__ logits, int t0, int M, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int lane) {
    if (E <= 64)
        router_rows16_nq<4>(logits, t0, M, E, k, ids, w, lane);
    else if (E <= 128)
        router_rows16_nq<8>(logits, t0, M, E, k, ids, w, lane);
    else
        router_rows16_nq<16>(logits, t0, M, E, k, ids, w, lane);
}

// Lanes holding the same expert id (9-bit ids; 0x1FF = no route).
__device__ __forceinline__ uint64_t same_expert(int e) {
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    return same;
}

}  // namespace moe
