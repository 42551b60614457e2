// stream_gemm.hip -- weight-streaming grouped FP8 GEMMs for batches with few
// tokens per expert (decode and verify).
//
// Each wave owns 16 weight rows of one expert and streams them once from HBM
// (K contiguous, 128 bytes per row per K block, fetched as whole lines by
// nontemporal loads (load_lines_nt: the weights are read once, so they are
// not kept in the caches) and turned into MFMA fragments through a 4 KiB LDS
// buffer per wave: 6-11% faster than per-lane fragment loads, measured), feeding
// v_mfma_f32_16x16x128 with the weights as the A
// operand and up to 16 of the expert's routes as the B operand (unused
// columns are zero).  One MFMA covers one 128-wide K block, so the block
// scales are applied per block: acc += blk * (s_act[token, kb] * s_w[e, n/128, kb])
// (Netra Kernel README capability table: explicit block-scale semantics).
//
// Gate/up writes FP32 results per route (Netra compiler architecture page:
// gate/up FP32).  Down starts by recomputing SiLU(gate) * up and its 1x128
// FP8 requantisation for its routes into LDS, then streams w2 the same way
// and writes one fp32 partial row per route (Netra Kernel README, MoE
// prefill pair: SiLU and quantisation, then down-partial).
#include "device.h"
#include "fused_decode.h"
#include "launch.h"

namespace moe {

constexpr int kRowsPerWave = 16;
constexpr int kWavesPerGroup = 4;
constexpr int kRowsPerGroup = kRowsPerWave * kWavesPerGroup;  // 64
// K blocks loaded per batch and wave.  Small batches keep the register
// count low, so more workgroups stay resident and more bytes are in flight
// per CU (measured on MI355X at h = 6144: 8 -> 4 cut gate/up time by 23%,
// 8 -> 2 cut down time by 34%; holding a whole down tile in registers ahead
// of the SiLU prologue was slower for the occupancy it costs).
constexpr int kUnrollUp = 4;
constexpr int kUnrollDown = 3;

// Gate/up batches: kUpBatch K blocks of the wave's weight lines in registers;
// the 16 routes' activation codes and scales of the batch copied once per
// workgroup straight into LDS (global_load_lds: one 1 KiB copy per route,
// four per wave, and one copy of their scales), two buffers, one barrier per
// batch.  With no activation operand held in registers, a batch of 8 blocks
// (16 KiB of weights per wave in flight) fits four waves per SIMD.
constexpr int kUpBatch = 8;
constexpr int kUpStageRow = 128 * kUpBatch + 16;   // one route's codes of a batch (padded: conflict-free reads)

__global__ __launch_bounds__(256) void stream_gate_up_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xs, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ active,
    const int32_t* __restrict__ num_active, float* __restrict__ g, int h, int i, int k) {
    const int slot = blockIdx.y;
    if (slot >= *num_active) return;
    const int e = active[slot];
    const int beg = offsets[e], cnt = offsets[e + 1] - beg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int N = 2 * i, KB = h / 128, nb = (KB + kUpBatch - 1) / kUpBatch;
    const int n0 = blockIdx.x * kRowsPerGroup + wave * kRowsPerWave;
    const int col = lane & 15, kg = lane >> 4;
    const uint8_t* wrow = w13 + ((size_t)e * N + n0) * h;
    const float* ws = s13 + ((size_t)e * (N / 128) + n0 / 128) * KB;
    __shared__ __align__(16) uint8_t bounce[kWavesPerGroup][2][2048];   // line-to-fragment buffers
    __shared__ __align__(16) uint8_t stage[2][16 * kUpStageRow];        // activation codes of a batch
    __shared__ __align__(16) float xsl[2][kWavesPerGroup][64];          // their scales: wave w's routes 4 w .. 4 w + 3

    for (int j0 = 0; j0 < cnt; j0 += 16) {
        const bool valid = j0 + col < cnt;
        const int p = valid ? sorted[beg + j0 + col] : 0;
        // the routes this wave copies (past the expert's routes: its first; its scale is never used)
        const uint8_t* xst[4];
        const float* xsst[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jr = j0 + 4 * wave + r;
            const int tr = (jr < cnt ? sorted[beg + jr] : sorted[beg]) / k;
            xst[r] = xq + (size_t)tr * h;
            xsst[r] = xs + (size_t)tr * KB;
        }
        const int lr = (lane & 31) >> 3;   // scale copy: route 4 wave + lr, block kb0 + lane % 8
        const float* xss = lr == 0 ? xsst[0] : lr == 1 ? xsst[1] : lr == 2 ? xsst[2] : xsst[3];
        v8i A[kUpBatch];
        float wsv[kUpBatch];
        // batch b into buffer bi: the activation codes and scales by copies,
        // the weight lines and scales into registers
        auto issue = [&](int b, int bi) {
            const int kb0 = b * kUpBatch;
            const int off = min(kb0 * 128 + 16 * lane, h - 16);   // past the last K block: never read
#pragma unroll
            for (int r = 0; r < 4; ++r)
                copy16_to_lds(xst[r] + off,
                              (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&stage[bi][(4 * wave + r) * kUpStageRow])));
            copy4_to_lds(xss + min(kb0 + (lane & 7), KB - 1),
                         (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&xsl[bi][wave][0])));
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                const int kb = kb0 + u;
                if (kb < KB) {
                    A[u] = load_lines_nt(wrow + kb * 128, h, lane);
                    wsv[u] = ws[kb];
                }
            }
        };
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        issue(0, 0);
        for (int b = 0; b < nb; ++b) {
            const int bi = b & 1;
            // this wave's copies and loads of the batch have landed; the barrier
            // publishes every wave's copies (and certifies that the other buffer
            // is no longer read)
            __builtin_amdgcn_s_waitcnt(vm_wait(0));
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                const int kb = b * kUpBatch + u;
                if (kb < KB) {
                    const v8i B = load32(&stage[bi][col * kUpStageRow + u * 128 + kg * 32]);
                    const float sc = valid ? xsl[bi][col >> 2][(col & 3) * 8 + u] * wsv[u] : 0.0f;
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f blk = mfma_16x16x128_e4m3(lines_to_frag(A[u], &bounce[wave][u & 1][0], lane, col, kg), B, z);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
                }
            }
            if (b + 1 < nb) issue(b + 1, bi ^ 1);
        }
        __syncthreads();   // the stage buffers are reused by the next group of routes
        if (valid)
            *reinterpret_cast<float4*>(g + (size_t)p * N + n0 + kg * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

// One route's gate and up values of one 128-column group, 8 columns per lane
// of a 16-lane row.
struct GateUp8 {
    float4 g0, g1, u0, u1;
};
__device__ __forceinline__ GateUp8 load_gate_up8(const float* __restrict__ gate, int sub, int i) {
    const float4* gp = reinterpret_cast<const float4*>(gate + sub * 8);
    const float4* up = reinterpret_cast<const float4*>(gate + i + sub * 8);
    return {gp[0], gp[1], up[0], up[1]};
}

// SiLU(gate) * up of one 128-column group for one route on one 16-lane row,
// requantised to E4M3 (amax over the row by DPP); stored only where live.
__device__ __forceinline__ void silu_quant_row(const GateUp8& x, int sub, uint8_t* __restrict__ q,
                                               float* __restrict__ s, bool write_scale, bool live = true) {
    const float a[8] = {x.g0.x, x.g0.y, x.g0.z, x.g0.w, x.g1.x, x.g1.y, x.g1.z, x.g1.w};
    const float b[8] = {x.u0.x, x.u0.y, x.u0.z, x.u0.w, x.u1.x, x.u1.y, x.u1.z, x.u1.w};
    float v[8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = (a[j] / (1.0f + expf(-a[j]))) * b[j];
        m = fmaxf(m, fabsf(v[j]));
    }
    m = row16_max(m);
    const float sc = m / kE4M3Max;
    const uint2 codes = quant8(v, sc);
    if (live) {
        *reinterpret_cast<uint2*>(q + sub * 8) = codes;
        if (write_scale) *s = sc;
    }
}

__host__ __device__ inline size_t stream_down_lds_base(int i) {
    return ((size_t)16 * (i + 16) + (size_t)16 * (i / 128) * 4 + 15) & ~(size_t)15;
}

__global__ __launch_bounds__(256) void stream_down_kernel(
    const float* __restrict__ g, const uint8_t* __restrict__ w2, const float* __restrict__ s2,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ active, const int32_t* __restrict__ num_active,
    float* __restrict__ y, int h, int i, int k) {
    extern __shared__ uint8_t lds[];
    const int slot = blockIdx.y;
    if (slot >= *num_active) return;
    const int e = active[slot];
    const int beg = offsets[e], cnt = offsets[e + 1] - beg;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int IB = i / 128;
    const int astride = i + 16;                         // padded LDS row of one route's codes
    uint8_t* a2l = lds;                                 // [16][astride]
    float* a2sl = reinterpret_cast<float*>(lds + 16 * astride);   // [16][IB]
    const int n0 = blockIdx.x * kRowsPerGroup + wave * kRowsPerWave;
    const int col = lane & 15, kg = lane >> 4;
    const uint8_t* wrow = w2 + ((size_t)e * h + n0) * i;
    const float* ws = s2 + ((size_t)e * (h / 128) + n0 / 128) * IB;
    uint8_t* bnc = lds + stream_down_lds_base(i) + wave * 4096;
    const int sub = lane & 15;

    for (int j0 = 0; j0 < cnt; j0 += 16) {
        const int nr = min(16, cnt - j0), ntask = nr * IB;
        __syncthreads();
        // The prologue's first task per 16-lane row (route jr, column group
        // b): its gate/up reads go out first, then the first weight batch, so
        // the weights stream while the SiLU codes are computed (the memory
        // counter retires in order: waiting for the gate/up values does not
        // wait for the weights issued after them).
        // (Both unconditional, with clamped indices, so that the compiler's
        // count of outstanding loads is the same on every path.)
        const int t0 = wave * 4 + (lane >> 4);
        const int tc = min(t0, ntask - 1), jr0 = tc / IB, b0 = tc - jr0 * IB;
        const GateUp8 x0 = load_gate_up8(g + (size_t)sorted[beg + j0 + jr0] * 2 * i + b0 * 128, sub, i);
        v8i A[kUnrollDown];
        float wsv[kUnrollDown];
        // The weight loads take a zero K-block offset that passes through an
        // empty asm here, so the compiler neither hoists the first batch out of
        // the route-group loop (ahead of the gate/up reads) nor moves it above
        // them.
        int kz = 0;
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" : "+s"(kz));
        // batch kb0's weight lines and scales (past the last K block: the last
        // block again, never used)
        auto load_w = [&](int kb0) {
#pragma unroll
            for (int u = 0; u < kUnrollDown; ++u) {
                const int kb = min(kb0 + u, IB - 1) + kz;
                A[u] = load_lines_nt(wrow + kb * 128, i, lane);
                wsv[u] = ws[kb];
            }
        };
        load_w(0);
        __builtin_amdgcn_sched_barrier(0);   // every request of the batch before the SiLU codes
        // (computed on every row, so that the gate/up loads stay in this block)
        silu_quant_row(x0, sub, a2l + jr0 * astride + b0 * 128, a2sl + jr0 * IB + b0, sub == 0, t0 < ntask);
        for (int task = t0 + 16; task < ntask; task += 16) {
            const int jr = task / IB, b = task - jr * IB;
            const GateUp8 x = load_gate_up8(g + (size_t)sorted[beg + j0 + jr] * 2 * i + b * 128, sub, i);
            silu_quant_row(x, sub, a2l + jr * astride + b * 128, a2sl + jr * IB + b, sub == 0);
        }
        __syncthreads();
        const bool valid = col < nr;
        const int p = valid ? sorted[beg + j0 + col] : 0;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb0 = 0; kb0 < IB; kb0 += kUnrollDown) {
            // As in gate/up: all loads of the batch first (the first batch's
            // before the prologue), scales multiplied in the MFMA loop.  The
            // activation codes are read from LDS for every column; a column
            // past the routes gets a zero scale.
            if (kb0 > 0) load_w(kb0);
            __builtin_amdgcn_sched_barrier(0);
            v8i B[kUnrollDown];
            float asv[kUnrollDown];
#pragma unroll
            for (int u = 0; u < kUnrollDown; ++u) {
                const int kb = kb0 + u;
                if (kb < IB) {
                    B[u] = valid ? load32(a2l + col * astride + kb * 128 + kg * 32) : zero8();
                    asv[u] = valid ? a2sl[col * IB + kb] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnrollDown; ++u) {
                const int kb = kb0 + u;
                if (kb < IB) {
                    const float sc = asv[u] * wsv[u];
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f blk = mfma_16x16x128_e4m3(lines_to_frag(A[u], bnc + (u & 1) * 2048, lane, col, kg), B[u], z);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(blk[v], sc, acc[v]);
                }
            }
        }
        if (valid)
            *reinterpret_cast<float4*>(y + (size_t)p * h + n0 + kg * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
}

hipError_t launch_stream_gate_up(const StreamArgs& a, const uint8_t* xq, const float* xs,
                                 const uint8_t* w13, const float* s13, float* g, hipStream_t stream) {
    const dim3 grid((2 * a.i) / kRowsPerGroup, a.max_slots);
    launch(stream_gate_up_kernel, grid, dim3(256), 0, stream, xq, xs, w13, s13, a.offsets,
                       a.sorted, a.active, a.num_active, g, a.h, a.i, a.k);
    return hipGetLastError();
}

static size_t stream_down_lds_bytes(int i) { return stream_down_lds_base(i) + 4 * 4096; }

hipError_t launch_stream_down(const StreamArgs& a, const float* g, const uint8_t* w2, const float* s2,
                              float* y, hipStream_t stream) {
    const dim3 grid(a.h / kRowsPerGroup, a.max_slots);
    launch(stream_down_kernel, grid, dim3(256), stream_down_lds_bytes(a.i), stream, g, w2,
                       s2, a.offsets, a.sorted, a.active, a.num_active, y, a.h, a.i, a.k);
    return hipGetLastError();
}

// ------------------------------------------------------------- combine

// out[t, n] = bf16( sum_{r < k} w[t, r] * y[t*k + r, n] ), r ascending,
// multiply then add, from 0 (Inferact amd-kernels README, atomics rule).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ tw, int k, int h,
                                                      uint16_t* __restrict__ out) {
#pragma clang fp contract(off)
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= h) return;
    // every rank's partial is requested before the rank-order sum starts
    v4f v[16];   // streaming loads: every partial is read once
    float w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r < k) {
            w[r] = tw[(size_t)t * k + r];
            v[r] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(y + ((size_t)t * k + r) * h + n));
        }
    }
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r < k) {
            a0 = a0 + w[r] * v[r][0];
            a1 = a1 + w[r] * v[r][1];
            a2 = a2 + w[r] * v[r][2];
            a3 = a3 + w[r] * v[r][3];
        }
    }
    *reinterpret_cast<uint2*>(out + (size_t)t * h + n) = make_uint2(bf16x2(a0, a1), bf16x2(a2, a3));
}

// The same combine over bf16 partials: eight columns per thread.
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ y,
                                                           const float* __restrict__ tw, int k, int h,
                                                           uint16_t* __restrict__ out, const uint32_t* err) {
#pragma clang fp contract(off)
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (n >= h) return;
    if (err != nullptr && (ld_agent(err) & kErrProducer) != 0u) {   // the producer gave up: NaN
        *reinterpret_cast<uint4*>(out + (size_t)t * h + n) = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
        return;
    }
    v4i v[16];   // streaming loads: every partial is read once
    float w[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r < k) {
            w[r] = tw[(size_t)t * k + r];
            v[r] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(y + ((size_t)t * k + r) * h + n));
        }
    }
    float a[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (r < k) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[2 * q] = a[2 * q] + w[r] * bf16_lo((uint32_t)v[r][q]);
                a[2 * q + 1] = a[2 * q + 1] + w[r] * bf16_hi((uint32_t)v[r][q]);
            }
        }
    }
    *reinterpret_cast<uint4*>(out + (size_t)t * h + n) =
        make_uint4(bf16x2(a[0], a[1]), bf16x2(a[2], a[3]), bf16x2(a[4], a[5]), bf16x2(a[6], a[7]));
}

hipError_t launch_combine_bf16(const uint16_t* y, const float* tw, int M, int k, int h, uint16_t* out,
                               hipStream_t stream, const uint32_t* err) {
    const dim3 grid((h / 8 + 255) / 256, M);
    launch(combine_bf16_kernel, grid, dim3(256), 0, stream, y, tw, k, h, out, err);
    return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* tw, int M, int k, int h, uint16_t* out,
                          hipStream_t stream) {
    const dim3 grid((h / 4 + 255) / 256, M);
    launch(combine_kernel, grid, dim3(256), 0, stream, y, tw, k, h, out);
    return hipGetLastError();
}

}  // namespace moe
