// front_end.hip -- the step before the layer's activation quantisation: an
// RMSNorm of bf16 rows fused with the 1x128 E4M3 quantisation (the gfx950
// "normalization and quantization fusions" family of the Netra Kernel README
// directory map), so x is read once and the layer's codes and scales come out
// of the same pass.
//
// Per row (readings of the pages, which name the fusion but not its
// arithmetic): ss = sum of x^2 with every square exact in float64; r =
// fp32(1 / sqrt(ss / h + eps)) evaluated in float64 and rounded once; y[c] =
// bf16_rne(fp32(fp32(x[c] * r) * gamma[c])); then the layer's activation
// quantisation of the bf16 row (scale amax/448 per 128 columns, codes
// E4M3(RN_fp32(y / s))).
//
// One wave per row: lane l holds columns 512 st + 8 l .. + 7 of every 512-
// column step st, so the 16 lanes of a DPP row cover one 128-column group
// (the same mapping as the layer's quantiser).  The whole row stays in
// registers between the sum of squares and the output (h <= 8192).  The
// float64 sum runs per lane over its columns, then over the wave by an xor
// butterfly, which leaves the identical total in every lane.
#include "device.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kFrontWaves = 4;                       // rows per workgroup
constexpr int kFrontMaxSteps = kFrontMaxHidden / 512;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// STEPS = ceil(h / 512) is a template parameter, so the row lives in
// registers and every loop unrolls.
template <int STEPS>
__global__ __launch_bounds__(kFrontWaves * kWave) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gamma, float eps, int M, int h,
    uint16_t* __restrict__ y, uint8_t* __restrict__ q, float* __restrict__ s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kFrontWaves + (threadIdx.x >> 6);
    if (row >= M) return;
    const uint16_t* xr = x + (size_t)row * h;

    // columns past h (only in a ragged last step) load column 0 and count as zero
    uint4 u[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int c = st * 512 + lane * 8;
        u[st] = *reinterpret_cast<const uint4*>(xr + (c < h ? c : 0));
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st)
        if (st * 512 + lane * 8 >= h) u[st] = make_uint4(0, 0, 0, 0);

    double ss = 0.0;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const uint32_t w[4] = {u[st].x, u[st].y, u[st].z, u[st].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double a = (double)bf16_lo(w[j]), b = (double)bf16_hi(w[j]);
            ss += a * a;
            ss += b * b;
        }
    }
    ss = wave_sum_f64(ss);
    const float r = (float)(1.0 / sqrt(ss / (double)h + (double)eps));

    uint8_t* qr = q + (size_t)row * h;
    float* sr = s + (size_t)row * (h / 128);
    uint16_t* yr = y ? y + (size_t)row * h : nullptr;
    const int sub = lane & 15;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int c = st * 512 + lane * 8;
        const bool live = c < h;
        const int cg = live ? c : 0;
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + cg);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + cg + 4);
        const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const uint32_t w[4] = {u[st].x, u[st].y, u[st].z, u[st].w};
        uint32_t yb[4];
        float v[8];
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float n0 = bf16_lo(w[j]) * r, n1 = bf16_hi(w[j]) * r;
            yb[j] = bf16x2(n0 * gm[2 * j], n1 * gm[2 * j + 1]);
            v[2 * j] = bf16_lo(yb[j]);
            v[2 * j + 1] = bf16_hi(yb[j]);
            a = fmaxf(a, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
        }
        a = row16_max(a);                            // the 16 lanes of one group
        const float sc = a / kE4M3Max;
        if (live) {
            if (yr) *reinterpret_cast<uint4*>(yr + c) = make_uint4(yb[0], yb[1], yb[2], yb[3]);
            *reinterpret_cast<uint2*>(qr + c) = quant8(v, sc);
            if (sub == 0) sr[c / 128] = sc;
        }
    }
}

template <int STEPS>
hipError_t launch_steps(const uint16_t* x, const float* gamma, float eps, int M, int h, uint16_t* y,
                        uint8_t* q, float* s, hipStream_t stream) {
    if (STEPS != (h + 511) / 512) return launch_steps<(STEPS < kFrontMaxSteps ? STEPS + 1 : STEPS)>(
        x, gamma, eps, M, h, y, q, s, stream);
    hipLaunchKernelGGL(rmsnorm_quant_kernel<STEPS>, dim3((M + kFrontWaves - 1) / kFrontWaves),
                       dim3(kFrontWaves * kWave), 0, stream, x, gamma, eps, M, h, y, q, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_quant(const uint16_t* x, const float* gamma, float eps, int M, int h,
                                uint16_t* y, uint8_t* q, float* s, hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    if (h <= 0 || h % 128 != 0 || h > kFrontMaxHidden) return hipErrorInvalidValue;
    return launch_steps<1>(x, gamma, eps, M, h, y, q, s, stream);
}

}  // namespace moe
