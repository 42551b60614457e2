// prefill_gemm.hip -- tiled grouped FP8 GEMMs for batches with many tokens
// per expert (prefill).
//
// Routes are grouped by expert (counts, offsets, routes sorted by expert then
// route id).  An M-tile is 128 consecutive sorted routes of one expert; the
// grouping pass also numbers every expert's M-tiles (mtile_off).
//
// gate/up: one workgroup per (M-tile, 128-column group jg).  Its weight tile
// is the 128 gate rows and the 128 up rows of group jg of w13[e] (256 x h),
// its activation tile the E4M3 rows of the tile's tokens.  Per 128-wide K
// block (one scale block) both tiles are staged through LDS (double
// buffered: the next block's global loads are in flight while the current
// one feeds the MFMAs), each wave computes a 64-route x (64 gate + 64 up)
// quarter with v_mfma_f32_16x16x128_f8f6f4 (weights as A, routes as B) and
// promotes every block with its two scales: acc += blk * (s_w * s_act)
// (Netra Kernel README capability table: explicit 128x128 block scales).
// Because the tile holds a whole 128-column group of both halves, the
// epilogue computes SiLU(gate) * up and its 1x128 E4M3 requantisation on the
// spot (Netra Kernel README, MoE prefill pair: gate/up then SiLU and
// quantisation in the producer) and writes the codes in sorted-route order.
//
// down: one workgroup per (M-tile, 256-row tile of w2[e]); same pipeline over
// K = i, fp32 partial rows written by route id (down-partial).
//
// Workgroups are handed to XCDs round-robin; the tile order gives each XCD a
// contiguous range of tiles, so the tiles that share an activation tile (and
// the M-tiles of one expert, which share weights) meet in the same L2.
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kPBM = 128;          // routes per tile
constexpr int kPBN = 256;          // weight rows per tile
constexpr int kLdsRow = 128 + 16;  // one 128-byte K block per row, padded

__device__ __forceinline__ int xcd_tile(int b, int nb) {
    const int per = nb / 8;   // the grid is a multiple of 8
    return (b % 8) * per + b / 8;
}

__device__ __forceinline__ v8i lds32(const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    const uint4 u0 = q[0], u1 = q[1];
    v8i r;
    r[0] = (int)u0.x; r[1] = (int)u0.y; r[2] = (int)u0.z; r[3] = (int)u0.w;
    r[4] = (int)u1.x; r[5] = (int)u1.y; r[6] = (int)u1.z; r[7] = (int)u1.w;
    return r;
}

// Expert owning M-tile mt: the largest e with mtile_off[e] <= mt.
__device__ __forceinline__ int tile_expert(const int32_t* __restrict__ mtile_off, int E, int mt) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (mtile_off[mid] <= mt) lo = mid; else hi = mid;
    }
    return lo;
}

// Staging of one 128-wide K block of a 256-row A tile and a 128-row B tile:
// thread t moves A chunks t + 256j (j < 8) and B chunks t + 256j (j < 4),
// chunk c = 16 bytes at row c / 8, column 16 * (c % 8).
struct Stage {
    uint4 ra[8];
    uint4 rb[4];
};

template <typename ARow, typename BRow>
__device__ __forceinline__ void stage_load(Stage& s, int tid, int kb, ARow arow, BRow brow) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = tid + 256 * j;
        s.ra[j] = *reinterpret_cast<const uint4*>(arow(c >> 3) + kb * 128 + (c & 7) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j;
        const uint8_t* src = brow(c >> 3);
        s.rb[j] = src ? *reinterpret_cast<const uint4*>(src + kb * 128 + (c & 7) * 16)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void stage_store(const Stage& s, int tid, uint8_t* As, uint8_t* Bs) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<uint4*>(As + (c >> 3) * kLdsRow + (c & 7) * 16) = s.ra[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<uint4*>(Bs + (c >> 3) * kLdsRow + (c & 7) * 16) = s.rb[j];
    }
}

// One K block on one wave: 8 weight tiles (rows wrow0[j] .. +16 of the LDS A
// tile) x 4 route tiles (rows wm*64 + 16m of the LDS B tile), promoted with
// scale ws[j] * xs[m].
__device__ __forceinline__ void block_mma(v4f acc[8][4], const uint8_t* As, const uint8_t* Bs,
                                          const int wrow0[8], int tok0, int col, int kg,
                                          const float ws[8], const float xsv[4]) {
    v8i B[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) B[m] = lds32(Bs + (tok0 + 16 * m + col) * kLdsRow + kg * 32);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const v8i A = lds32(As + (wrow0[j] + col) * kLdsRow + kg * 32);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
            const v4f blk = mfma_16x16x128_e4m3(A, B[m], z);
            const float sc = ws[j] * xsv[m];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[j][m][v] = fmaf(blk[v], sc, acc[j][m][v]);
        }
    }
}

// ----------------------------------------------------------------- gate/up

__global__ __launch_bounds__(256, 1) void prefill_gate_up_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int h = a.h, i = a.i, E = a.E, k = a.k;
    const int KB = h / 128, IB = i / 128, N13 = 2 * i;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;

    const int L = xcd_tile(blockIdx.x, gridDim.x);
    const int mt = L / IB, jg = L - mt * IB;
    if (mt >= a.mtile_off[E]) return;
    const int e = tile_expert(a.mtile_off, E, mt);
    const int beg = a.offsets[e] + (mt - a.mtile_off[e]) * kPBM;
    const int rows = min(kPBM, a.offsets[e + 1] - beg);

    uint8_t* As = smem;                                          // [2][256][kLdsRow]
    uint8_t* Bs = As + 2 * kPBN * kLdsRow;                       // [2][128][kLdsRow]
    int* tok_l = reinterpret_cast<int*>(Bs + 2 * kPBM * kLdsRow);  // [128] token, -1 = padding
    float* amax_l = reinterpret_cast<float*>(tok_l + kPBM);      // [2][128]
    float* xs_l = amax_l + 2 * kPBM;                             // [128][KB]

    for (int r = tid; r < kPBM; r += 256) tok_l[r] = r < rows ? a.sorted[beg + r] / k : -1;
    __syncthreads();
    for (int idx = tid; idx < kPBM * KB; idx += 256) {
        const int r = idx / KB, kb = idx - r * KB;
        const int t = tok_l[r];
        xs_l[idx] = t >= 0 ? a.xs[(size_t)t * KB + kb] : 0.0f;
    }

    const uint8_t* wbase = a.w13 + (size_t)e * N13 * h;
    auto arow = [&](int r) {   // LDS row r: gate rows of group jg, then up rows
        const int wr = r < 128 ? jg * 128 + r : i + jg * 128 + (r - 128);
        return wbase + (size_t)wr * h;
    };
    auto brow = [&](int r) -> const uint8_t* {
        const int t = tok_l[r];
        return t >= 0 ? a.xq + (size_t)t * h : nullptr;
    };
    const float* sg = a.s13 + ((size_t)e * (N13 / 128) + jg) * KB;
    const float* su = a.s13 + ((size_t)e * (N13 / 128) + IB + jg) * KB;

    int wrow0[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wrow0[j] = (j < 4 ? 0 : 128) + wn * 64 + 16 * (j & 3);
    const int tok0 = wm * 64;

    v4f acc[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[j][m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    Stage st;
    stage_load(st, tid, 0, arow, brow);
    stage_store(st, tid, As, Bs);
    __syncthreads();
    for (int kb = 0; kb < KB; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < KB) stage_load(st, tid, kb + 1, arow, brow);
        float ws[8], xsv[4];
        const float g = sg[kb], u = su[kb];
#pragma unroll
        for (int j = 0; j < 8; ++j) ws[j] = j < 4 ? g : u;
#pragma unroll
        for (int m = 0; m < 4; ++m) xsv[m] = xs_l[(tok0 + 16 * m + col) * KB + kb];
        block_mma(acc, As + cur * kPBN * kLdsRow, Bs + cur * kPBM * kLdsRow, wrow0, tok0, col, kg,
                  ws, xsv);
        if (kb + 1 < KB) stage_store(st, tid, As + (cur ^ 1) * kPBN * kLdsRow,
                                     Bs + (cur ^ 1) * kPBM * kLdsRow);
        __syncthreads();
    }

    // ---- epilogue: SiLU(gate) * up, 1x128 requantisation of group jg.
    // Lane: route tok0 + 16m + col; gate/up columns wn*64 + 16jj + 4kg + v.
    float pm[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        pm[m] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float gt = acc[jj][m][v], up = acc[jj + 4][m][v];
                const float val = (gt / (1.0f + expf(-gt))) * up;
                acc[jj][m][v] = val;
                pm[m] = fmaxf(pm[m], fabsf(val));
            }
        pm[m] = fmaxf(pm[m], __shfl_xor(pm[m], 16, kWave));
        pm[m] = fmaxf(pm[m], __shfl_xor(pm[m], 32, kWave));
        if (kg == 0) amax_l[wn * kPBM + tok0 + 16 * m + col] = pm[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = tok0 + 16 * m + col;
        if (r >= rows) continue;
        const float sc = fmaxf(amax_l[r], amax_l[kPBM + r]) / kE4M3Max;
        const size_t pos = (size_t)(beg + r);
        uint32_t* dst = reinterpret_cast<uint32_t*>(a.a2 + pos * i + jg * 128 + wn * 64 + 4 * kg);
        const float rc = sc != 0.0f ? __builtin_amdgcn_rcpf(sc) : 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const uint32_t q = sc == 0.0f ? 0u
                : quant4(acc[jj][m][0], acc[jj][m][1], acc[jj][m][2], acc[jj][m][3], sc, rc);
            dst[4 * jj] = q;   // columns wn*64 + 16jj + 4kg .. +3
        }
        if (wn == 0 && kg == 0) a.a2s[pos * IB + jg] = sc;
    }
}

// -------------------------------------------------------------------- down

__global__ __launch_bounds__(256, 1) void prefill_down_kernel(PrefillArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int h = a.h, i = a.i, E = a.E;
    const int IB = i / 128, NT = h / kPBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;

    const int L = xcd_tile(blockIdx.x, gridDim.x);
    const int mt = L / NT, nt = L - mt * NT;
    if (mt >= a.mtile_off[E]) return;
    const int e = tile_expert(a.mtile_off, E, mt);
    const int beg = a.offsets[e] + (mt - a.mtile_off[e]) * kPBM;
    const int rows = min(kPBM, a.offsets[e + 1] - beg);

    uint8_t* As = smem;
    uint8_t* Bs = As + 2 * kPBN * kLdsRow;
    int* prt_l = reinterpret_cast<int*>(Bs + 2 * kPBM * kLdsRow);   // [128] route id, -1 = padding
    float* xs_l = reinterpret_cast<float*>(prt_l + kPBM);         // [128][IB]

    for (int r = tid; r < kPBM; r += 256) prt_l[r] = r < rows ? a.sorted[beg + r] : -1;
    for (int idx = tid; idx < kPBM * IB; idx += 256) {
        const int r = idx / IB, kb = idx - r * IB;
        xs_l[idx] = r < rows ? a.a2s[(size_t)(beg + r) * IB + kb] : 0.0f;
    }
    __syncthreads();

    const uint8_t* wbase = a.w2 + ((size_t)e * h + (size_t)nt * kPBN) * i;
    auto arow = [&](int r) { return wbase + (size_t)r * i; };
    auto brow = [&](int r) -> const uint8_t* {
        return r < rows ? a.a2 + (size_t)(beg + r) * i : nullptr;
    };
    // the wave's 128 weight rows lie in one 128-row scale block
    const float* sw = a.s2 + ((size_t)e * (h / 128) + (nt * kPBN + wn * 128) / 128) * IB;

    int wrow0[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wrow0[j] = wn * 128 + 16 * j;
    const int tok0 = wm * 64;

    v4f acc[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[j][m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    Stage st;
    stage_load(st, tid, 0, arow, brow);
    stage_store(st, tid, As, Bs);
    __syncthreads();
    for (int kb = 0; kb < IB; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < IB) stage_load(st, tid, kb + 1, arow, brow);
        float ws[8], xsv[4];
        const float w = sw[kb];
#pragma unroll
        for (int j = 0; j < 8; ++j) ws[j] = w;
#pragma unroll
        for (int m = 0; m < 4; ++m) xsv[m] = xs_l[(tok0 + 16 * m + col) * IB + kb];
        block_mma(acc, As + cur * kPBN * kLdsRow, Bs + cur * kPBM * kLdsRow, wrow0, tok0, col, kg,
                  ws, xsv);
        if (kb + 1 < IB) stage_store(st, tid, As + (cur ^ 1) * kPBN * kLdsRow,
                                     Bs + (cur ^ 1) * kPBM * kLdsRow);
        __syncthreads();
    }

    // ---- epilogue: fp32 partial rows by route id
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = tok0 + 16 * m + col;
        const int p = prt_l[r];
        if (p < 0) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float* dst = a.y + (size_t)p * h + nt * kPBN + wrow0[j] + 4 * kg;
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[j][m][0], acc[j][m][1], acc[j][m][2], acc[j][m][3]);
        }
    }
}

static size_t gate_up_lds(int h) {
    return (size_t)2 * (kPBN + kPBM) * kLdsRow + kPBM * 4 + 2 * kPBM * 4 + (size_t)kPBM * (h / 128) * 4;
}
static size_t down_lds(int i) {
    return (size_t)2 * (kPBN + kPBM) * kLdsRow + kPBM * 4 + (size_t)kPBM * (i / 128) * 4;
}

int prefill_tile_m() { return kPBM; }

bool prefill_supported(int h, int i) {
    return h % kPBN == 0 && i % 128 == 0 && gate_up_lds(h) <= 160 * 1024 && down_lds(i) <= 160 * 1024;
}

static int round8(int v) { return (v + 7) / 8 * 8; }

hipError_t launch_prefill(const PrefillArgs& a, int R, hipStream_t stream) {
    static bool configured = false;
    if (!configured) {
        hipFuncSetAttribute((const void*)prefill_gate_up_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        hipFuncSetAttribute((const void*)prefill_down_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        configured = true;
    }
    const int max_mt = R / kPBM + a.E;   // >= sum over experts of ceil(count / 128)
    const int g1 = round8(max_mt * (a.i / 128));
    hipLaunchKernelGGL(prefill_gate_up_kernel, dim3(g1), dim3(256), gate_up_lds(a.h), stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int g2 = round8(max_mt * (a.h / kPBN));
    hipLaunchKernelGGL(prefill_down_kernel, dim3(g2), dim3(256), down_lds(a.i), stream, a);
    return hipGetLastError();
}

}  // namespace moe
