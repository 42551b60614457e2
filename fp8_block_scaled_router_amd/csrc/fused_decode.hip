// fused_decode.hip -- the whole layer in one persistent kernel for small
// batches (M <= 16 tokens): decode and speculative verification.
//
// Every workgroup first recomputes, on chip, what it needs from the batch:
// the router top-k of all M tokens (one wave per token, DPP/cross-lane
// argmax), the 1x128 E4M3 activation codes of all tokens (into LDS) and the
// grouping of the M*k routes by expert (ballot ranks).  Nothing then stands
// between the kernel start and the first weight load but the logits and x
// reads.  Work is split in two task lists:
//
//  A task (expert slot u, 128-column group jg, quarter q): 32 gate rows and
//    the matching 32 up rows of w13[e_u], K = h, streamed once with
//    v_mfma_f32_16x16x128_f8f6f4 (weights as A, the expert's <= 16 routes as
//    B), per-128-K-block scale promotion; FP32 results per route (Netra
//    compiler architecture page: gate/up FP32).  A ticket counts the four
//    quarters of (u, jg); the last one computes SiLU(gate) * up for the
//    group and requantises it to E4M3 per 128 columns (Netra Kernel README,
//    MoE prefill pair: SiLU and quantisation), then counts the group done.
//  B task (expert slot u, 64-row tile of w2[e_u]): loads its weights into
//    registers before it waits for expert u's activations, then computes the
//    fp32 partial rows of u's routes (down-partial).  A ticket per (token,
//    tile) counts the token's k routes; the last one sums the k partials in
//    rank order and writes bf16 (route reducer; Inferact amd-kernels README,
//    atomics rule: atomics only count, sums run in a fixed order).
//
// Synchronisation words live at the start of the workspace.  They must be
// zero before the first forward and every forward leaves them zero (the last
// arriver of each ticket resets it, the last workgroup to exit resets the
// done counters).  Waits are bounded in time; a timeout sets a sticky error
// word instead of hanging.  The grid never exceeds the number of workgroups
// that can be resident at once, so every awaited task is always running.
#include "device.h"
#include "fused_decode.h"

namespace moe {

constexpr int kFusedMaxM = 16;
constexpr int kFusedMaxIB = 8;              // i <= 1024
constexpr int kQuarters = 4;                // A task: 32 gate + 32 up rows
constexpr int kDownRows = 64;               // B task rows
constexpr uint64_t kWaitTicks = 100000000;  // 1 s of the 100 MHz constant clock

// ---------------------------------------------------------------------
// routing of one token on one wave, results to LDS

__device__ __forceinline__ void route_token(const float* __restrict__ l, int E, int k,
                                            int* ids_l, float* w_l, int lane) {
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        key[j] = (e < E) ? float_order_key(l[e]) : 0u;
    }
    int picked[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        picked[r] = 0;
        if (r < k) {
            uint32_t hi = 0u, lo = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (key[j] > hi) {
                    hi = key[j];
                    lo = 0xFFFFu - (uint32_t)(lane + 64 * j);
                }
            }
            wave_key_max(hi, lo);
            int e = (int)(0xFFFFu - lo);
            e = (hi == 0u || e >= E) ? E - 1 : e;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (lane + 64 * j == e) key[j] = 0u;
            picked[r] = e;
        }
    }
    const float lmax = l[picked[0]];
    float ex[16];
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        ex[r] = 0.0f;
        if (r < k) {
            ex[r] = expf(l[picked[r]] - lmax);
            sum += ex[r];
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r < k && lane == r) {
            ids_l[r] = picked[r];
            w_l[r] = ex[r] / sum;
        }
    }
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
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

__device__ __forceinline__ void silu_quant_group(const float* __restrict__ gate,
                                                 const float* __restrict__ up, int sub,
                                                 uint8_t* __restrict__ q, float* __restrict__ s) {
    const float4 g0 = reinterpret_cast<const float4*>(gate + sub * 8)[0];
    const float4 g1 = reinterpret_cast<const float4*>(gate + sub * 8)[1];
    const float4 u0 = reinterpret_cast<const float4*>(up + sub * 8)[0];
    const float4 u1 = reinterpret_cast<const float4*>(up + sub * 8)[1];
    const float a[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float b[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float v[8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = (a[j] / (1.0f + expf(-a[j]))) * b[j];
        m = fmaxf(m, fabsf(v[j]));
    }
    m = row16_max(m);
    const float sc = m / kE4M3Max;
    *reinterpret_cast<uint2*>(q + sub * 8) = quant8(v, sc);
    if (sub == 0) *s = sc;
}

// Thread 0 waits until *ctr >= target (bounded), then the workgroup acquires.
__device__ __forceinline__ void wait_count(uint32_t* ctr, uint32_t target, uint32_t* err) {
    if (threadIdx.x == 0) {
        const uint64_t t0 = wall_clock64();
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (wall_clock64() - t0 > kWaitTicks) {
                atomicOr(err, 1u);
                break;
            }
        }
    }
    __syncthreads();
    __threadfence();
}

__global__ __launch_bounds__(256) void fused_decode_kernel(FusedArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int M = a.M, h = a.h, i = a.i, E = a.E, k = a.k;
    const int R = M * k, G = h / 128, IB = i / 128, KB = h / 128, N13 = 2 * i;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;

    // ---- LDS carve (all offsets 16-byte aligned)
    uint8_t* xq_l = smem;                                            // [M][h]
    float* xs_l = reinterpret_cast<float*>(xq_l + M * h);            // [M][G]
    int* ids_l = reinterpret_cast<int*>(xs_l + ((M * G + 3) & ~3));  // [R]
    float* w_l = reinterpret_cast<float*>(ids_l + ((R + 3) & ~3));   // [R]
    int* off_l = reinterpret_cast<int*>(w_l + ((R + 3) & ~3));       // [E+1]
    int* act_l = off_l + ((E + 1 + 3) & ~3);                         // [E]
    int* srt_l = act_l + ((E + 3) & ~3);                             // [R]
    int* base_l = srt_l + ((R + 3) & ~3);                            // [E]
    int* misc_l = base_l + ((E + 3) & ~3);                           // [32]
    uint8_t* a2_l = reinterpret_cast<uint8_t*>(misc_l + 32);         // [16][i + 16]
    const int a2_stride = i + 16;
    float* a2s_l = reinterpret_cast<float*>(a2_l + 16 * a2_stride);  // [16][IB]

    // ---- phase 0: routing, activation codes and grouping, on every workgroup
    for (int t = wave; t < M; t += 4)
        route_token(a.logits + (size_t)t * E, E, k, ids_l + t * k, w_l + t * k, lane);
    for (int task = wave * 4 + (lane >> 4); task < M * G; task += 16) {
        const int t = task / G, g = task - t * G;
        const uint4 u = *reinterpret_cast<const uint4*>(a.x + (size_t)t * h + g * 128 + col * 8);
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
    __syncthreads();
    if (wave == 0) {
        // counts per expert (lane owns experts 4l..4l+3), then offsets and the
        // ascending list of experts with routes
        for (int e = lane; e < E; e += 64) base_l[e] = 0;
        for (int p0 = 0; p0 < R; p0 += 64) {
            const int p = p0 + lane;
            const int e = p < R ? ids_l[p] : 0x1FF;
            const uint64_t same = match_id(e);
            if (p < R && (same >> lane) == 1ull) base_l[e] += __popcll(same);
        }
        int tot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[j] = (4 * lane + j < E) ? base_l[4 * lane + j] : 0;
        const int lsum = tot[0] + tot[1] + tot[2] + tot[3];
        const int lact = (tot[0] > 0) + (tot[1] > 0) + (tot[2] > 0) + (tot[3] > 0);
        const int incl = wave_incl_scan_i(lsum, lane);
        const int iact = wave_incl_scan_i(lact, lane);
        int run = incl - lsum, arun = iact - lact;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            if (e < E) {
                off_l[e] = run;
                base_l[e] = run;
                if (tot[j] > 0) act_l[arun] = e;
            }
            run += tot[j];
            arun += (tot[j] > 0);
        }
        if (lane == 63) {
            off_l[E] = incl;
            misc_l[0] = iact;
        }
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int p0 = 0; p0 < R; p0 += 64) {
            const int p = p0 + lane;
            const int e = p < R ? ids_l[p] : 0x1FF;
            const uint64_t same = match_id(e);
            int pos = 0;
            if (p < R) pos = base_l[e] + __popcll(same & below);
            if (p < R) {
                srt_l[pos] = p;
                if ((same >> lane) == 1ull) base_l[e] += __popcll(same);
            }
        }
    }
    __syncthreads();
    const int U = misc_l[0];

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

    // ---- phase 1: gate/up quarters
    const int nA = U * IB * kQuarters;
    for (int task = blockIdx.x; task < nA; task += gridDim.x) {
        const int u = task / (IB * kQuarters);
        const int rem = task - u * IB * kQuarters;
        const int jg = rem / kQuarters, q = rem - jg * kQuarters;
        const int e = act_l[u];
        const int beg = off_l[e], cnt = off_l[e + 1] - beg;
        const int row0 = (wave >> 1) * i + jg * 128 + q * 32 + (wave & 1) * 16;
        const uint8_t* wrow = a.w13 + ((size_t)e * N13 + row0 + col) * h + kg * 32;
        const float* ws = a.s13 + ((size_t)e * (N13 / 128) + row0 / 128) * KB;
        const bool valid = col < cnt;
        const int p = valid ? srt_l[beg + col] : 0;
        const int t = p / k;
        const uint8_t* xrow = xq_l + t * h + kg * 32;
        const float* xsr = xs_l + t * G;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb0 = 0; kb0 < KB; kb0 += 8) {
            v8i A[8];
            float ws8[8];
#pragma unroll
            for (int u8 = 0; u8 < 8; ++u8) {
                if (kb0 + u8 < KB) {
                    A[u8] = load32(wrow + (kb0 + u8) * 128);
                    ws8[u8] = ws[kb0 + u8];
                }
            }
#pragma unroll
            for (int u8 = 0; u8 < 8; ++u8) {
                const int kb = kb0 + u8;
                if (kb < KB) {
                    const v8i B = valid ? load32(xrow + kb * 128) : zero8();
                    const float sc = (valid ? xsr[kb] : 0.0f) * ws8[u8];
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f blk = mfma_16x16x128_e4m3(A[u8], B, z);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
                }
            }
        }
        if (valid)
            *reinterpret_cast<float4*>(a.g + (size_t)p * N13 + row0 + kg * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = atomicAdd(a.gate_tix + u * IB + jg, 1u);
            misc_l[1] = (old == kQuarters - 1);
        }
        __syncthreads();
        if (misc_l[1]) {
            __threadfence();
            for (int jr = wave * 4 + (lane >> 4); jr < cnt; jr += 16) {
                const int pr = srt_l[beg + jr];
                const float* gr = a.g + (size_t)pr * N13 + jg * 128;
                silu_quant_group(gr, gr + i, col, a.a2 + (size_t)pr * i + jg * 128,
                                 a.a2s + (size_t)pr * IB + jg);
            }
            __threadfence();
            __syncthreads();
            if (tid == 0) {
                __hip_atomic_store(a.gate_tix + u * IB + jg, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                atomicAdd(a.done + u, 1u);
            }
        }
        __syncthreads();
    }

    // ---- phase 2: down tiles, then the fixed-order combine
    const int NT = h / kDownRows;
    const int nB = U * NT;
    for (int task = blockIdx.x; task < nB; task += gridDim.x) {
        const int u = task / NT, nt = task - u * NT;
        const int e = act_l[u];
        const int beg = off_l[e], cnt = off_l[e + 1] - beg;
        const int n0 = nt * kDownRows + wave * 16;
        const uint8_t* wrow = a.w2 + ((size_t)e * h + n0 + col) * i + kg * 32;
        const float* ws = a.s2 + ((size_t)e * (h / 128) + n0 / 128) * IB;
        v8i W[kFusedMaxIB];
        float ws8[kFusedMaxIB];
#pragma unroll
        for (int kb = 0; kb < kFusedMaxIB; ++kb) {
            if (kb < IB) {
                W[kb] = load32(wrow + kb * 128);
                ws8[kb] = ws[kb];
            }
        }
        wait_count(a.done + u, (uint32_t)IB, a.err);
        for (int idx = tid; idx < cnt * (i / 16); idx += 256) {
            const int jr = idx / (i / 16), c16 = idx - jr * (i / 16);
            const int pr = srt_l[beg + jr];
            *reinterpret_cast<uint4*>(a2_l + jr * a2_stride + c16 * 16) =
                *reinterpret_cast<const uint4*>(a.a2 + (size_t)pr * i + c16 * 16);
        }
        for (int idx = tid; idx < cnt * IB; idx += 256) {
            const int jr = idx / IB, b = idx - jr * IB;
            a2s_l[jr * IB + b] = a.a2s[(size_t)srt_l[beg + jr] * IB + b];
        }
        __syncthreads();
        const bool valid = col < cnt;
        const int p = valid ? srt_l[beg + col] : 0;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < kFusedMaxIB; ++kb) {
            if (kb < IB) {
                const v8i B = valid ? load32(a2_l + col * a2_stride + kb * 128 + kg * 32) : zero8();
                const float sc = (valid ? a2s_l[col * IB + kb] : 0.0f) * ws8[kb];
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f blk = mfma_16x16x128_e4m3(W[kb], B, z);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
            }
        }
        if (valid)
            *reinterpret_cast<float4*>(a.y + (size_t)p * h + n0 + kg * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        __threadfence();
        __syncthreads();
        if (tid < cnt) {
            const int pr = srt_l[beg + tid];
            const int t = pr / k;
            const uint32_t old = atomicAdd(a.comb_tix + t * NT + nt, 1u);
            misc_l[2 + tid] = (old == (uint32_t)(k - 1)) ? t : -1;
        }
        __syncthreads();
        bool any = false;
        for (int jr = 0; jr < cnt; ++jr) any |= misc_l[2 + jr] >= 0;
        if (any) {
            __threadfence();
            for (int jr = 0; jr < cnt; ++jr) {
                const int t = misc_l[2 + jr];
                if (t < 0) continue;
                if (tid < kDownRows) {
#pragma clang fp contract(off)
                    const int n = nt * kDownRows + tid;
                    float accum = 0.0f;
                    for (int r = 0; r < k; ++r)
                        accum = accum + w_l[t * k + r] * a.y[((size_t)t * k + r) * h + n];
                    __bf16 b = (__bf16)accum;
                    a.out[(size_t)t * h + n] = __builtin_bit_cast(uint16_t, b);
                }
                if (tid == 0)
                    __hip_atomic_store(a.comb_tix + t * NT + nt, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }

    // ---- exit: the last workgroup resets the done counters
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(a.exit_cnt, 1u);
        if (old == gridDim.x - 1) {
            for (int u = 0; u < a.umax; ++u)
                __hip_atomic_store(a.done + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.exit_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __threadfence();
        }
    }
}

size_t fused_lds_bytes(int M, int h, int i, int E, int k) {
    const int R = M * k, G = h / 128, IB = i / 128;
    auto r4 = [](int v) { return (size_t)((v + 3) & ~3); };
    size_t b = (size_t)M * h;
    b += r4(M * G) * 4;
    b += r4(R) * 4 * 2;
    b += r4(E + 1) * 4 + r4(E) * 4 + r4(R) * 4 + r4(E) * 4 + 32 * 4;
    b += (size_t)16 * (i + 16) + (size_t)16 * IB * 4;
    return (b + 15) & ~(size_t)15;
}

bool fused_supported(int M, int h, int i, int E, int k) {
    return M >= 1 && M <= kFusedMaxM && k <= 16 && E <= 256 && h % 128 == 0 && i % 128 == 0 &&
           i / 128 <= kFusedMaxIB && (size_t)M * h <= 32768 && h % kDownRows == 0 &&
           (size_t)M * (h / kDownRows) <= 2048 && fused_lds_bytes(M, h, i, E, k) <= 64 * 1024;
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
    const int want = std::max(args.umax * IB * kQuarters, args.umax * (args.h / kDownRows));
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
