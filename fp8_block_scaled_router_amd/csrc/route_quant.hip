// route_quant.hip -- router top-k and per-token 1x128 FP8 activation
// quantisation (gfx950, wave64).
//
// Router (Netra Kernel README capability table, "BF16 routing" family;
// kernel-laboratory README, decode and verification routing kernels): a
// token's logits are spread over a wave (experts lane + 64q) or over a
// 16-lane row (experts lane + 16q); each lane sorts its own candidates once,
// and each of the k rounds takes the largest head key of the group, the
// lowest expert among the heads that reach it (so equal logits go to the
// lower expert index, and -0 equals +0), and pops that head.  The weights are
// exp(l - l_max) of the picks divided by their sum in rank order (the full
// softmax denominator cancels in the renormalisation).
//
// Activation quantisation (Netra compiler architecture page: FP8 activation
// with fp32 activation-scale tensors): one 16-lane DPP row per 128-column
// group, eight bf16 per lane from one 16-byte load; amax by a DPP row
// reduction, s = amax / 448, q = E4M3(x / s).
#include "device.h"
#include "launch.h"
#include "route_quant.h"

namespace moe {

// Four tokens per workgroup of five waves: wave 4 routes the four tokens
// (router_rows16) while waves 0-3 quantise one row each.
constexpr int kRouteQuantThreads = 5 * kWave;
__global__ __launch_bounds__(kRouteQuantThreads) void route_quant_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int h,
    int32_t* __restrict__ ids, float* __restrict__ tw, uint8_t* __restrict__ xq,
    float* __restrict__ xs, int what) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = blockIdx.x * 4;
    if (wave == 4) {
        if (what & kRoute) router_rows16(logits, t0, M, E, k, ids, tw, lane);
        return;
    }
    const int t = t0 + wave;
    if (t >= M) return;
    if (what & kQuant)
        act_quant_row(x + (size_t)t * h, h, xq + (size_t)t * h, xs + (size_t)t * (h / 128), 0, 1, lane);
}

hipError_t launch_route_quant(const float* logits, const uint16_t* x, int M, int E, int k, int h,
                              int32_t* ids, float* tw, uint8_t* xq, float* xs, int what,
                              hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    launch(route_quant_kernel, dim3((M + 3) / 4), dim3(kRouteQuantThreads), 0, stream, logits, x, M, E, k, h,
                       ids, tw, xq, xs, what);
    return hipGetLastError();
}

// Router, activation quantisation and grouping in one launch, for batches of
// at most kGroupTailRoutes routes.  Each workgroup routes and quantises one
// token; its ids go out with device-coherent stores, then it counts itself
// in.  The last workgroup to arrive groups every route on one wave (ballot
// matches give each route's rank inside its expert in route order, DPP
// prefix sums the offsets and the active list) and resets the counter.  No
// workgroup ever waits for another.
__global__ __launch_bounds__(256) void route_quant_group_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int E, int k, int h,
    int32_t* __restrict__ ids, float* __restrict__ tw, uint8_t* __restrict__ xq, float* __restrict__ xs,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active, uint32_t* arrivals) {
    __shared__ int cnt_l[256];
    __shared__ int last_l;
    const int t = blockIdx.x, M = gridDim.x, R = M * k;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint4 u[kQuantBatch];   // the row's first loads are in flight while wave 0 routes
    act_quant_load(x + (size_t)t * h, h, 0, wave, 4, lane, u);
    if (wave == 0) router_wave(logits + (size_t)t * E, E, k, ids + (size_t)t * k, tw + (size_t)t * k, lane, true);
    act_quant_finish(x + (size_t)t * h, h, xq + (size_t)t * h, xs + (size_t)t * (h / 128), wave, 4, lane, u);
    if (tid == 0) {
        wait_vmem();   // this wave's id stores have completed
        last_l = atomicAdd(arrivals, 1u) == (uint32_t)(M - 1);
    }
    __syncthreads();
    if (!last_l || wave != 0) return;

    for (int e = lane; e < E; e += 64) cnt_l[e] = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int lr[4], ee[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        lr[b] = 0;
        ee[b] = 0x1FF;
        if (64 * b < R) {
            const int p = 64 * b + lane;
            const int e = p < R ? (int)ld_agent(reinterpret_cast<const uint32_t*>(ids) + p) : 0x1FF;
            const uint64_t same = same_expert(e);
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
    const int lact = (c[0] > 0) + (c[1] > 0) + (c[2] > 0) + (c[3] > 0);
    const int incl = wave_scan_incl(lsum);
    const int iact = wave_scan_incl(lact);
    int run = incl - lsum, arun = iact - lact;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        if (e < E) {
            cnt_l[e] = run;   // becomes the offset
            offsets[e] = run;
            counts[e] = c[j];
            if (c[j] > 0) active[arun] = e;
        }
        run += c[j];
        arun += (c[j] > 0);
    }
    if (lane == 63) {
        offsets[E] = incl;
        *num_active = iact;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int p = 64 * b + lane;
        if (p < R) sorted[cnt_l[ee[b]] + lr[b]] = p;
    }
    if (lane == 0) st_agent(arrivals, 0u);
}

hipError_t launch_route_quant_group(const float* logits, const uint16_t* x, int M, int E, int k, int h,
                                    int32_t* ids, float* tw, uint8_t* xq, float* xs, int32_t* counts,
                                    int32_t* offsets, int32_t* sorted, int32_t* active,
                                    int32_t* num_active, uint32_t* arrivals, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if ((int64_t)M * k > kGroupTailRoutes || E > 256) return hipErrorInvalidValue;
    launch(route_quant_group_kernel, dim3(M), dim3(256), 0, stream, logits, x, E, k, h, ids,
                       tw, xq, xs, counts, offsets, sorted, active, num_active, arrivals);
    return hipGetLastError();
}

// ------------------------------------------------ BF16 routing logits + top-k
//
// BF16 routing (Netra Kernel README capability table; Inferact amd-kernels
// README, routing entries): logits[t][e] = sum_j x[t][j] * wr[e][j] over bf16
// hidden rows and a bf16 router weight, then the top-k of step 1 on those
// logits, in one launch.  Each workgroup takes 32 tokens (two 16-row MFMA
// fragments) and every expert; its four waves split K (wave w takes the
// 128-column steps w, w + 4, ...), so each wave streams a quarter of the
// router weight with all of a step's loads in flight at once.  A lane reads
// 32 contiguous bytes of its row per load pair, so the four lanes of a row
// cover whole 128-byte lines.  v_mfma_f32_16x16x32_bf16 accumulates in fp32:
// every bf16 product is exact in fp32, the additions are not (the oracle
// rounds a float64 sum once).  The four partial tiles are added in LDS in wave
// order, each element by one thread (deterministic), the 32 x E logits go out to `logits` when asked, and
// router_rows16 routes the 32 tokens from LDS, four per wave per pass.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kRgTokens = 32;

__device__ __forceinline__ v4f mfma_16x16x32_bf16(const uint4& a, const uint4& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                   0, 0, 0);
}

// 16 bytes of a row at element offset k0 + 64 p + 8 hf + 16 q (the lane's
// piece u = 2 p + hf of a 128-column step); A and B use the same positions.
__device__ __forceinline__ void load_step(const uint16_t* __restrict__ rowq, int k0, uint4 f[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) f[u] = *reinterpret_cast<const uint4*>(rowq + k0 + 64 * (u >> 1) + 8 * (u & 1));
}

// NFMAX: expert fragments the template holds (E <= 16 * NFMAX), loaded eight
// at a time per step.
template <int NFMAX>
__global__ __launch_bounds__(256) void router_gemm_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int M, int h, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ tw) {
    __shared__ float part[4][kRgTokens * 16 * NFMAX];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * kRgTokens;
    const int Ml = min(kRgTokens, M - t0);
    const int NF = (E + 15) >> 4;
    const int nsteps = h / 128;

    // Rows past M or E read a live row instead; their results are dropped.
    const uint16_t* xp[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int t = t0 + 16 * m + row;
        xp[m] = x + (size_t)(t < M ? t : t0) * h + 16 * q;
    }
    v4f acc[2][NFMAX];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < NFMAX; ++j) acc[m][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int st = wave; st < nsteps; st += 4) {
        const int k0 = 128 * st;
        uint4 a[2][4];
        load_step(xp[0], k0, a[0]);
        load_step(xp[1], k0, a[1]);
#pragma unroll
        for (int c = 0; c < NFMAX; c += 8) {
            if (c < NF) {
                uint4 b[8][4];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int e = 16 * (c + j) + row;
                    load_step(wr + (size_t)(e < E ? e : 0) * h + 16 * q, k0, b[j]);
                }
                // Keep every load of the step ahead of the first MFMA: left to
                // itself the scheduler sinks each load to its use and the step
                // becomes a chain of dependent memory round trips.
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
#pragma unroll
                        for (int m = 0; m < 2; ++m)
                            acc[m][c + j] = mfma_16x16x32_bf16(a[m][u], b[j][u], acc[m][c + j]);
            }
        }
    }
    // Lane (row, q) of tile (m, j) holds expert 16 j + row of tokens
    // 16 m + 4 q + v.  Each wave stores its partial tile, then every thread
    // adds the four partials of its elements in wave order.
#pragma unroll
    for (int j = 0; j < NFMAX; ++j) {
        const int e = 16 * j + row;
        if (e < E)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) part[wave][(16 * m + 4 * q + v) * E + e] = acc[m][j][v];
    }
    __syncthreads();
    float* lg = part[0];
    for (int idx = tid; idx < kRgTokens * E; idx += 256)
        lg[idx] = ((part[0][idx] + part[1][idx]) + part[2][idx]) + part[3][idx];
    __syncthreads();
    if (logits)
        for (int idx = tid; idx < Ml * E; idx += 256) logits[(size_t)t0 * E + idx] = lg[idx];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int tl = 16 * pass + 4 * wave;
        if (tl < Ml) router_rows16(lg, tl, Ml, E, k, ids + (size_t)t0 * k, tw + (size_t)t0 * k, lane);
    }
}

// The same logits for few tokens, spread over the experts: workgroup
// (token tile, expert fragment f) computes 32 tokens x experts 16 f .. 16 f + 15
// and stores them to `logits`; the row router then runs as a second launch.
// Each logit follows the arithmetic of router_gemm_topk_kernel exactly (wave w
// sums the steps w, w + 4, ... in ascending order, four MFMAs per step, and the
// four partials are added in wave order), so both paths give the same bits.
// A wave issues the loads of up to three of its steps before their MFMAs.
__global__ __launch_bounds__(256) void router_logits_split_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr, int M, int h,
                                                                  int E, float* __restrict__ logits) {
    __shared__ float part[4][kRgTokens * 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * kRgTokens, f = blockIdx.y;
    const int Ml = min(kRgTokens, M - t0);
    const int nsteps = h / 128;
    const uint16_t* xp[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int t = t0 + 16 * m + row;
        xp[m] = x + (size_t)(t < M ? t : t0) * h + 16 * q;
    }
    const int e = 16 * f + row;
    const uint16_t* wp = wr + (size_t)(e < E ? e : 0) * h + 16 * q;
    v4f acc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
    for (int st0 = wave; st0 < nsteps; st0 += 12) {
        uint4 a[3][2][4], b[3][4];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int k0 = 128 * min(st0 + 4 * r, nsteps - 1);
            load_step(xp[0], k0, a[r][0]);
            load_step(xp[1], k0, a[r][1]);
            load_step(wp, k0, b[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 3; ++r)
            if (st0 + 4 * r < nsteps)
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int m = 0; m < 2; ++m) acc[m] = mfma_16x16x32_bf16(a[r][m][u], b[r][u], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wave][(16 * m + 4 * q + v) * 16 + row] = acc[m][v];
    __syncthreads();
    for (int idx = tid; idx < kRgTokens * 16; idx += 256) {
        const int t = idx >> 4, ee = 16 * f + (idx & 15);
        if (t < Ml && ee < E)
            logits[(size_t)(t0 + t) * E + ee] = ((part[0][idx] + part[1][idx]) + part[2][idx]) + part[3][idx];
    }
}

// Token tiles below which the experts are spread over workgroups (when the
// caller keeps the logits): under it the fused kernel would leave most CUs
// idle while one workgroup per tile streams the whole router weight.
constexpr int kRgSplitTiles = 128;

hipError_t launch_router_gemm_topk(const uint16_t* x, const uint16_t* wr, int M, int h, int E, int k,
                                   float* logits, int32_t* ids, float* tw, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if (E < 1 || E > 256 || h % 128 != 0) return hipErrorInvalidValue;
    const int tiles = (M + kRgTokens - 1) / kRgTokens;
    if (logits && tiles < kRgSplitTiles) {
        hipLaunchKernelGGL(router_logits_split_kernel, dim3(tiles, (E + 15) / 16), dim3(256), 0, stream, x, wr, M, h,
                           E, logits);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        return launch_route_quant(logits, nullptr, M, E, k, 128, ids, tw, nullptr, nullptr, kRoute, stream);
    }
    const dim3 grid(tiles), block(256);
    if (E <= 128)
        hipLaunchKernelGGL(router_gemm_topk_kernel<8>, grid, block, 0, stream, x, wr, M, h, E, k, logits, ids, tw);
    else
        hipLaunchKernelGGL(router_gemm_topk_kernel<16>, grid, block, 0, stream, x, wr, M, h, E, k, logits, ids, tw);
    return hipGetLastError();
}

// ------------------------------------------------------------ utilities

__global__ __launch_bounds__(256) void encode_e4m3_kernel(const float* __restrict__ in, int64_t n,
                                                          uint8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; j < n; j += stride) {
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const int m = (n - j) < 4 ? (int)(n - j) : 4;
        for (int u = 0; u < m; ++u) v[u] = in[j + u];
        const uint32_t c = e4m3x4(v[0], v[1], v[2], v[3]);
        for (int u = 0; u < m; ++u) out[j + u] = (uint8_t)(c >> (8 * u));
    }
}

hipError_t launch_encode_e4m3(const float* in, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 1023) / 1024;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(encode_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, n, out);
    return hipGetLastError();
}

// One workgroup per 128x128 block: amax, s = amax / 448, codes E4M3(w / s).
__global__ __launch_bounds__(256) void quant_weight_kernel(const float* __restrict__ w, int N, int K,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ s) {
    const int NB = N / 128, KB = K / 128;
    const int64_t blk = blockIdx.x;
    const int64_t b = blk / ((int64_t)NB * KB);
    const int nb = (int)((blk / KB) % NB), kb = (int)(blk % KB);
    const int tid = threadIdx.x;
    const int row = tid >> 1, col0 = (tid & 1) * 64;
    const float* src = w + ((b * N + (int64_t)nb * 128 + row) * K) + (int64_t)kb * 128 + col0;
    uint8_t* dst = q + ((b * N + (int64_t)nb * 128 + row) * K) + (int64_t)kb * 128 + col0;
    float v[64];
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const float4 f = reinterpret_cast<const float4*>(src)[u];
        v[4 * u] = f.x; v[4 * u + 1] = f.y; v[4 * u + 2] = f.z; v[4 * u + 3] = f.w;
        a = fmaxf(a, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
    a = row16_max(a);
    a = xor16_max(a);
    a = xor32_max(a);
    __shared__ float part[4];
    if ((tid & 63) == 0) part[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float sc = a / kE4M3Max;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        uint2 c0 = quant8(&v[16 * u], sc);
        uint2 c1 = quant8(&v[16 * u + 8], sc);
        reinterpret_cast<uint4*>(dst)[u] = make_uint4(c0.x, c0.y, c1.x, c1.y);
    }
    if (tid == 0) s[blk] = sc;
}

hipError_t launch_quant_weight(const float* w, int64_t batch, int N, int K, uint8_t* q, float* s,
                               hipStream_t stream) {
    const int64_t blocks = batch * (N / 128) * (K / 128);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K, q,
                       s);
    return hipGetLastError();
}

}  // namespace moe
