// device.h -- device-side building blocks shared by the gfx950 kernels of
// the routed FP8 MoE layer: E4M3 / bf16 conversion, 16-lane DPP reductions,
// the FP8 MFMA tile and vector load helpers.  Wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
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

// E4M3 codes of four values v / s, exactly E4M3(RN_fp32(v / s)) (the
// correctly rounded fp32 quotient, then E4M3 rounding), without a division
// on the common path.  q = v * rcp(s) is within 2^-22 (relative) of v / s
// (v_rcp_f32 is accurate to 1 ulp), so RN_fp32(v / s) lies strictly between
// q * (1 - 2^-20) and q * (1 + 2^-20).  E4M3 rounding is monotone: when both
// ends give the same code, that is the code of RN_fp32(v / s).  Otherwise
// (v / s within a hair of an E4M3 rounding boundary) the exact division
// decides.  Tiny scales, whose reciprocal could overflow, take the division.
__device__ __forceinline__ uint32_t quant4(float v0, float v1, float v2, float v3, float s,
                                           float r) {
    const float lo = 1.0f - 0x1.0p-20f, hi = 1.0f + 0x1.0p-20f;
    const float q0 = v0 * r, q1 = v1 * r, q2 = v2 * r, q3 = v3 * r;
    const uint32_t a = e4m3x4(q0 * lo, q1 * lo, q2 * lo, q3 * lo);
    const uint32_t b = e4m3x4(q0 * hi, q1 * hi, q2 * hi, q3 * hi);
    if (__builtin_expect(a == b && s >= 0x1.0p-100f, 1)) return a;
    return e4m3x4(v0 / s, v1 / s, v2 / s, v3 / s);
}

// Quantise eight floats that share the scale s (s == 0 gives zero codes):
// codes E4M3(RN_fp32(v / s)).
__device__ __forceinline__ uint2 quant8(const float v[8], float s) {
    uint2 c;
    if (s == 0.0f) {
        c.x = 0u;
        c.y = 0u;
    } else {
        const float r = __builtin_amdgcn_rcpf(s);
        c.x = quant4(v[0], v[1], v[2], v[3], s, r);
        c.y = quant4(v[4], v[5], v[6], v[7], s, r);
    }
    return c;
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

// gfx950 row swaps with both operands v: for every lane, the two halves of
// the result are v of rows (2q, 2q + 1) (permlane16) or of rows (q, q + 2)
// (permlane32) at the lane's position, so one VALU instruction (no LDS
// crossbar) gives each lane its partner row's value.
__device__ __forceinline__ void key_step_rows16(uint32_t& hi, uint32_t& lo) {
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    hi = h[0];
    lo = l[0];
    key_max(hi, lo, h[1], l[1]);
}
__device__ __forceinline__ void key_step_rows32(uint32_t& hi, uint32_t& lo) {
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    hi = h[0];
    lo = l[0];
    key_max(hi, lo, h[1], l[1]);
}
// Max of v over lanes l, l ^ 16 (and l ^ 32) for v >= 0 (amax reductions).
__device__ __forceinline__ float xor16_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Inclusive prefix sum over the 64 lanes, DPP only: shifts of 1, 2, 4, 8
// inside each row of 16, then the row totals carried by row_bcast:15 and
// row_bcast:31.
__device__ __forceinline__ int wave_scan_incl(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

// Unsigned max over the 16 lanes of each DPP row.
__device__ __forceinline__ uint32_t row16_max_u(uint32_t v) {
    v = max(v, dpp_u<kDppQuadXor1>(v));
    v = max(v, dpp_u<kDppQuadXor2>(v));
    v = max(v, dpp_u<kDppRowHalfMirror>(v));
    v = max(v, dpp_u<kDppRowMirror>(v));
    return v;
}

// Wave-wide lexicographic max of 64-bit keys: DPP inside each row of 16
// lanes, then the two row swaps.  Every lane gets the result.
__device__ __forceinline__ void wave_key_max(uint32_t& hi, uint32_t& lo) {
    key_step_dpp<kDppQuadXor1>(hi, lo);
    key_step_dpp<kDppQuadXor2>(hi, lo);
    key_step_dpp<kDppRowHalfMirror>(hi, lo);
    key_step_dpp<kDppRowMirror>(hi, lo);
    key_step_rows16(hi, lo);
    key_step_rows32(hi, lo);
}

// Order-preserving map of an fp32 value to an unsigned key; -0 and +0 map to
// the same key.  Larger float -> larger key; all keys are nonzero for
// non-NaN inputs (0 is free to mean "no candidate").
__device__ __forceinline__ uint32_t float_order_key(float v) {
    if (v == 0.0f) v = 0.0f;
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of float_order_key (for a key of +-0 it returns +0).
__device__ __forceinline__ float float_from_order_key(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// ------------------------------------------- exchange between workgroups
//
// Data handed from one workgroup to another goes through agent-coherent
// stores and loads (relaxed agent-scope atomics: sc1, visible across the
// XCDs' separate L2s), and a writer waits for its own stores to complete
// before the workgroup counts a ticket.  This orders exactly the exchanged
// words without the whole-L2 write-back and invalidation an agent-scope fence
// costs on gfx950.

__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A value with the tag of the forward that wrote it, in one 64-bit word
// (stored and loaded whole, so a reader sees either the old word or the new).
__device__ __forceinline__ uint64_t ll_pack(float v, uint32_t tag) {
    return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}
__device__ __forceinline__ float ll_value(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t ll_tag(uint64_t w) { return (uint32_t)(w >> 32); }

// Thread 0 of a workgroup: waits until the device-scope word *ctr reaches
// n, with a growing sleep between polls, for at most 1 s of the 100 MHz
// constant clock.  Returns false when the wait timed out; `bit` is then set
// in the sticky error word *err.
__device__ __forceinline__ bool wait_count(const uint32_t* ctr, uint32_t n, uint32_t* err, uint32_t bit) {
    constexpr uint64_t kTicks = 100000000;
    uint64_t t0 = 0;
    int nap = 1;
    for (int tries = 0;; ++tries) {
        if (ld_agent(ctr) >= n) return true;
        if (tries == 0) t0 = wall_clock64();
        if (wall_clock64() - t0 > kTicks) {
            atomicOr(err, bit);
            return false;
        }
        for (int z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(2);
        nap = nap < 8 ? 2 * nap : 8;
    }
}

// Wait until every vector-memory operation this wave issued has completed
// (s_waitcnt vmcnt(0)); the signal fences keep the compiler from moving
// memory operations across it.
__device__ __forceinline__ void wait_vmem() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ----------------------------------------------------------------- MFMA

// D = A(16x128 e4m3) * B(128x16 e4m3) + C on gfx950.  Operand layout: lane l
// supplies row (l % 16) of A and column (l % 16) of B, each as 32 bytes that
// hold the same 32 K positions ("K slot group" l / 16).  Result: lane l
// holds column l % 16, rows 4 * (l / 16) + v for v = 0..3.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same instruction with an MXFP4 A operand: lane l (row l % 16, group
// g = l / 16) supplies 32 E2M1 codes (K elements 32 g .. 32 g + 31, element
// 2j in the low nibble of byte j) and their one E8M0 scale scale_a; B is the
// E4M3 operand in the layout the instruction takes for FP8 (lane group g
// holds K elements 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15) with
// its scale fixed at 1 (E8M0 127).
__device__ __forceinline__ v4f mfma_16x16x128_fp4_e4m3(const uint4& a, const v8i& b, int scale_a, const v4f& c) {
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4, 0, 0, scale_a, 0, 127);
}

// D = A(32x64) * B(64x32) + C, e4m3.  Lane l supplies row/column l % 32 and
// K slot group l / 32 (32 bytes); result lane l holds column l % 32, rows
// 8 * (v / 4) + 4 * (l / 32) + (v % 4) for v = 0..15.
__device__ __forceinline__ v16f mfma_32x32x64_e4m3(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Row r of a 16-row fragment holds its 32-byte K group kg as two 16-byte
// halves: the lower half in slot lo_slot(r, kg), the upper in lo_slot ^ 4.
// A fragment read (lane l: row l % 16, group l / 16) is then free of bank
// conflicts whether the LDS serves 8, 16 or 32 lanes of a ds_read_b128 at a
// time: every 8 consecutive rows of one kg fill the 8 slots of a 128-byte
// window, the 8 rows of one parity fill a 256-byte window, and the rows
// r, r + 4, r + 8, r + 12 of two adjacent groups fill the 8 slots of their
// 128-byte quarter of a 512-byte window.  Because only the slot, not the
// order of the two halves, depends on the row, every lane sees its K bytes
// in the same order.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) | (((r ^ (r >> 3)) & 1) << 2); }
__device__ __forceinline__ int lo_slot(int r, int kg) {
    const int x = swz(r);
    return (kg ^ (x & 3)) | (x & 4);
}
// Inverse: 16-byte K chunk (2 * kg + upper) stored in slot p of row r.
__device__ __forceinline__ int chunk_of(int r, int p) {
    const int x = swz(r);
    return 2 * ((p & 3) ^ (x & 3)) + (((p ^ x) >> 2) & 1);
}


// A 16-row weight tile fetched as whole 128-byte lines (8 lanes per line:
// lane l loads the chunk chunk_of(r, l % 8) of row r = l / 8, and of row
// 8 + l / 8); a stream of such loads touches 8 lines per instruction instead
// of the 16 half-used lines of per-lane fragment loads.  lines_to_frag turns
// the lines into the lane's MFMA fragment through a wave-private 2 KiB LDS
// buffer (contiguous writes, swizzled conflict-free reads; the wave's LDS
// operations stay in program order, so no barrier is needed).  The fragment
// bytes are those a direct fragment load would give.
__device__ __forceinline__ v8i load_lines(const uint8_t* __restrict__ row0, size_t stride, int lane) {
    const int r = lane >> 3, p = lane & 7;
    const uint4 x0 = *reinterpret_cast<const uint4*>(row0 + (size_t)r * stride + chunk_of(r, p) * 16);
    const uint4 x1 = *reinterpret_cast<const uint4*>(row0 + (size_t)(r + 8) * stride + chunk_of(r + 8, p) * 16);
    return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}
// The same tile with nontemporal loads (the weights of a decode forward are
// read once and need not stay in the caches).
__device__ __forceinline__ v8i load_lines_nt(const uint8_t* __restrict__ row0, size_t stride, int lane) {
    const int r = lane >> 3, p = lane & 7;
    const v4i x0 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(row0 + (size_t)r * stride + chunk_of(r, p) * 16));
    const v4i x1 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(row0 + (size_t)(r + 8) * stride + chunk_of(r + 8, p) * 16));
    return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}
__device__ __forceinline__ v8i lines_to_frag(const v8i& w, uint8_t* buf, int lane, int col, int kg) {
    *reinterpret_cast<uint4*>(buf + lane * 16) = make_uint4((uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]);
    *reinterpret_cast<uint4*>(buf + 1024 + lane * 16) = make_uint4((uint32_t)w[4], (uint32_t)w[5], (uint32_t)w[6], (uint32_t)w[7]);
    const int lo = lo_slot(col, kg);
    const uint4 u0 = *reinterpret_cast<const uint4*>(buf + col * 128 + lo * 16);
    const uint4 u1 = *reinterpret_cast<const uint4*>(buf + col * 128 + (lo ^ 4) * 16);
    return v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
}
__device__ __forceinline__ v8i load32(const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 u0 = q[0], u1 = q[1];
    v8i r;
    r[0] = (int)u0.x; r[1] = (int)u0.y; r[2] = (int)u0.z; r[3] = (int)u0.w;
    r[4] = (int)u1.x; r[5] = (int)u1.y; r[6] = (int)u1.z; r[7] = (int)u1.w;
    return r;
}

// gfx9 s_waitcnt immediate waiting until at most n vector-memory operations
// are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// global -> LDS copies (global_load_lds: no register receives the data).
// Written as inline assembly so that the compiler does not track them: a
// kernel that uses them waits for them itself (an explicit s_waitcnt before
// the barrier that publishes the bytes), and the compiler's own waits for
// later loads count only those loads (the hardware counter still retires in
// issue order, so a wave should issue its copies after the loads it needs
// first).  M0 holds the wave's LDS destination; lane l's data lands at
// M0 + 16 l (4 l for the dword form).  One wait state separates the M0
// write from the copy.
// kCoh: the copy reads at device scope (sc1), so it sees data that another
// workgroup of the same launch wrote with device-scope stores, whatever
// this XCD's L2 holds.
template <bool kCoh = false>
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds) {
    if constexpr (kCoh)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1"
                     :: "s"(lds), "v"(src) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(lds), "v"(src) : "memory", "m0");
}
template <bool kCoh = false>
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds) {
    if constexpr (kCoh)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off sc1"
                     :: "s"(lds), "v"(src) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                     :: "s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ v8i zero8() {
    v8i r;
    for (int j = 0; j < 8; ++j) r[j] = 0;
    return r;
}

}  // namespace moe
