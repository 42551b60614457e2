// device.h -- device-side building blocks shared by the gfx950 kernels of
// the routed FP8 MoE layer: E4M3 / bf16 conversion, 16-lane DPP reductions,
// the FP8 MFMA tile and vector load helpers.  Wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- formats

// E4M3 (OCP FN) conversion of four floats into one dword, byte j = value j.
// The hardware conversion rounds to nearest even; the clamp to +-448 makes it
// saturating (a quotient x / (amax/448) can exceed 448 by an fp32 ulp).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
    b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
    c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
    d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> two bf16 (round to nearest even, hardware), packed lo | hi << 16.
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Quantise eight floats that share the scale s (s == 0 gives zero codes).
// The quotient is the correctly rounded fp32 division v / s.
__device__ __forceinline__ uint2 quant8(const float v[8], float s) {
    uint2 r;
    if (s == 0.0f) {
        r.x = 0u;
        r.y = 0u;
    } else {
        r.x = e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
        r.y = e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    }
    return r;
}

// ------------------------------------------------------------ reductions

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;   // lane i <-> 15 - i inside a row of 16
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i inside each half row

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Max over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return v;
}

// Lexicographic max of (hi, lo) pairs.
__device__ __forceinline__ void key_max(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
    bool take = (ohi > hi) || (ohi == hi && olo > lo);
    hi = take ? ohi : hi;
    lo = take ? olo : lo;
}

template <int CTRL>
__device__ __forceinline__ void key_step_dpp(uint32_t& hi, uint32_t& lo) {
    uint32_t ohi = dpp_u<CTRL>(hi), olo = dpp_u<CTRL>(lo);
    key_max(hi, lo, ohi, olo);
}

__device__ __forceinline__ void key_step_xor(uint32_t& hi, uint32_t& lo, int mask) {
    uint32_t ohi = (uint32_t)__shfl_xor((int)hi, mask, kWave);
    uint32_t olo = (uint32_t)__shfl_xor((int)lo, mask, kWave);
    key_max(hi, lo, ohi, olo);
}

// Wave-wide lexicographic max of 64-bit keys: DPP inside each row of 16
// lanes, then two cross-row exchanges.  Every lane gets the result.
__device__ __forceinline__ void wave_key_max(uint32_t& hi, uint32_t& lo) {
    key_step_dpp<kDppQuadXor1>(hi, lo);
    key_step_dpp<kDppQuadXor2>(hi, lo);
    key_step_dpp<kDppRowHalfMirror>(hi, lo);
    key_step_dpp<kDppRowMirror>(hi, lo);
    key_step_xor(hi, lo, 16);
    key_step_xor(hi, lo, 32);
}

// Order-preserving map of an fp32 value to an unsigned key; -0 and +0 map to
// the same key.  Larger float -> larger key; all keys are nonzero for
// non-NaN inputs (0 is free to mean "no candidate").
__device__ __forceinline__ uint32_t float_order_key(float v) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------- MFMA

// D = A(16x128 e4m3) * B(128x16 e4m3) + C on gfx950.  Operand layout: lane l
// supplies row (l % 16) of A and column (l % 16) of B, each as 32 bytes that
// hold the same 32 K positions ("K slot group" l / 16).  Result: lane l
// holds column l % 16, rows 4 * (l / 16) + v for v = 0..3.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A(32x64) * B(64x32) + C, e4m3.  Lane l supplies row/column l % 32 and
// K slot group l / 32 (32 bytes); result lane l holds column l % 32, rows
// 8 * (v / 4) + 4 * (l / 32) + (v % 4) for v = 0..15.
__device__ __forceinline__ v16f mfma_32x32x64_e4m3(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 u0 = q[0], u1 = q[1];
    v8i r;
    r[0] = (int)u0.x; r[1] = (int)u0.y; r[2] = (int)u0.z; r[3] = (int)u0.w;
    r[4] = (int)u1.x; r[5] = (int)u1.y; r[6] = (int)u1.z; r[7] = (int)u1.w;
    return r;
}

__device__ __forceinline__ v8i zero8() {
    v8i r;
    for (int j = 0; j < 8; ++j) r[j] = 0;
    return r;
}

}  // namespace moe
