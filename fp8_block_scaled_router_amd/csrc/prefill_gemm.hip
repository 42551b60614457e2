// prefill_gemm.hip -- tiled grouped GEMMs with FP8 (128x128 block-scaled) or
// MXFP4 weights and E4M3 activations, for batches with many tokens per expert
// (prefill).
//
// Routes are grouped by expert (counts, offsets, routes sorted by expert then
// route id).  An M-tile is 128 consecutive sorted routes of one expert; the
// grouping pass also numbers every expert's M-tiles (mtile_off).
//
// gate/up tiles are (M-tile, 128-column group jg): the weight tile is the 128
// gate rows and the 128 up rows of group jg of w13[e] (256 x h), the
// activation tile the E4M3 rows of the tile's tokens.  down tiles are
// (M-tile, 256-row tile of w2[e]) over K = i.  Both kernels are persistent:
// one workgroup per CU walks the tiles of its XCD's share.
//
// Both kernels share one main loop, built for gfx950:
//  * 8 waves; each owns 64 weight rows x 64 routes = 4 x 4 tiles of
//    v_mfma_f32_16x16x128_f8f6f4 (weights as A, routes as B), two waves per
//    SIMD so one wave's promotion arithmetic overlaps the other's MFMAs.
//  * Every 128-wide K block (one scale block) of both operand tiles (48 KiB)
//    is copied global -> LDS by global_load_lds_dwordx4 (no register
//    staging) into one of three stage buffers: two blocks are in flight while
//    the third feeds the MFMAs.
//  * LDS rows are 128 bytes with a 16-byte-slot swizzle that keeps each
//    lane's 32 K bytes in order and spreads the 16 rows of a fragment over
//    all banks (lo_slot / chunk_of in device.h).
//  * The next tile's route list and scales are copied straight into LDS
//    during the current K loop, and its first two K blocks are issued before
//    the current tile's epilogue.
//  * Promotion with the two block scales (Netra Kernel README, capability
//    table: explicit 128x128 block scales): acc += blk * (s_w * s_act) in
//    fp32, one K block after the MFMA that produced blk, so the promotion
//    arithmetic never waits on an MFMA result.
// MXFP4 weights (the _mx_ kernels; Inferact amd-kernels README, naming
// section: moe/mxfp4_h6144_i768_e128_top4) take the same loop: 64-byte LDS
// weight rows (E2M1 codes of one K block) plus each row's four E8M0 scale
// bytes, copied beside them; the FP4 x FP8 form of the same MFMA applies the
// weight scales itself, and the promotion carries the activation scale alone.
// That form issues at the FP8 rate, so the loop's MFMA time is unchanged and
// only the weight copies halve.
// gate/up's epilogue computes SiLU(gate) * up and its 1x128 E4M3
// requantisation on the spot (Netra Kernel README, MoE prefill pair) and
// writes codes in sorted-route order; down writes bf16 partial rows by route
// id (the down-partial of the same README).
//
// Workgroups are handed to XCDs round-robin; each XCD's workgroups walk a
// contiguous range of tiles, so the M-tiles of one expert (which share its
// weights) meet in the same L2.
#include <algorithm>

#include "device.h"
#include "fused_decode.h"
#include "group.h"
#include "launch.h"
#include "route_quant.h"

namespace moe {
namespace {

constexpr int kBM = 128;                      // routes per tile
constexpr int kBN = 256;                      // weight rows per tile
constexpr int kThreads = 512;                 // 8 waves
constexpr int kBB = kBM * 128;                // activation bytes per stage
constexpr int kXS = 8 * 256;                  // activation scales per stage: 256 B per wave, 64 used
constexpr int kDmaB = kBB / 1024 / 8;         // 1 KiB activation copies per wave per stage
constexpr int kMaxKB = 128;                   // scale tables: K blocks (h, i <= 16384)

// Stage layout per weight format.  FP8 weights: 128 bytes per row and K
// block, fp32 128x128 block scales applied in the promotion.  MXFP4 weights
// (E2M1 codes two per byte, one E8M0 scale per 32 K elements): 64 bytes per
// row and K block, plus the rows' four scale bytes per K block, which the
// MFMA applies itself.
template <bool kMx>
struct Fmt {
    static constexpr int kRowBytes = kMx ? 64 : 128;       // weight bytes per row per K block
    static constexpr int kAB = kBN * kRowBytes;            // weight bytes per stage
    static constexpr int kAS = kMx ? 8 * 256 : 0;          // E8M0 scale words: 256 B per wave, 32 rows used
    static constexpr int kBOff = kAB + kAS;                // activation tile
    static constexpr int kXOff = kBOff + kBB;              // activation scales
    static constexpr int kStage = kXOff + kXS;
    static constexpr int kDmaA = kAB / 1024 / 8;           // 1 KiB weight copies per wave per stage
    // copies per wave per stage: weights, activations, 16 route scales, and
    // (MXFP4) 32 rows' scale words
    static constexpr int kVmem = kDmaA + kDmaB + 1 + (kMx ? 1 : 0);
};

static_assert(Fmt<false>::kDmaA == 4 && Fmt<true>::kDmaA == 2 && kDmaB == 2, "stage copy split");



// Per-tile routing metadata, staged in LDS with one coalesced load so a
// tile's set-up costs one global round trip instead of a chain of dependent
// ones.
constexpr int kMaxE = 256;
struct TileMeta {
    int mtile_off[kMaxE + 1];   // first M-tile of each expert
    int offsets[kMaxE + 1];     // first sorted route of each expert
};

// kCoh: the lists were written by other workgroups of the same launch.
template <bool kCoh = false>
__device__ __forceinline__ void load_meta(TileMeta& m, const PrefillArgs& a, int tid) {
    for (int j = tid; j <= a.E; j += kThreads) {
        m.mtile_off[j] = ld_i32<kCoh>(a.mtile_off + j);
        m.offsets[j] = ld_i32<kCoh>(a.offsets + j);
    }
}

// LDS of a tiled kernel: the ring of three stage buffers, the tile lists (per
// tile parity) and the epilogue's row maxima.  The producer runs both GEMMs
// on it in turn and uses the ring as scratch for its routing and grouping.
// (The small lists come first: their addresses then fit the DS
// instructions' 16-bit offsets.)
template <bool kMx>
struct TileLds {
    int rt[2][kBM];             // route id of each row (padding rows repeat the last route)
    float amax[4][kBM];         // gate/up epilogue: row maxima of the four column quarters
    float sw[2][2 * kMaxKB];    // FP8 weight scales: gate then up per K block, or the down tile's two row blocks
    TileMeta meta;
    int flag;                   // producer: this workgroup gives up the forward (a wait timed out)
    int last;                   // producer: this workgroup is the last to finish
    alignas(16) uint8_t stages[3 * Fmt<kMx>::kStage];
};

// Expert owning M-tile mt: the largest e with mtile_off[e] <= mt.
__device__ __forceinline__ int tile_expert(const int* mtile_off, int E, int mt) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (mtile_off[mid] <= mt) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ v8i frag(const uint8_t* lo, const uint8_t* hi) {
    const uint4 u0 = *reinterpret_cast<const uint4*>(lo);
    const uint4 u1 = *reinterpret_cast<const uint4*>(hi);
    v8i r;
    r[0] = (int)u0.x; r[1] = (int)u0.y; r[2] = (int)u0.z; r[3] = (int)u0.w;
    r[4] = (int)u1.x; r[5] = (int)u1.y; r[6] = (int)u1.z; r[7] = (int)u1.w;
    return r;
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// State of the shared main loop: wave-uniform bases (scalar registers) and
// 32-bit per-lane offsets (the prefill path is only taken when activation
// and requantised tensors stay below 2 GiB).
struct Loop {
    const uint8_t* gA;              // weight copies of K block 0 start here ...
    const uint8_t* gB;              // ... activation copies here
    const float* gX;                // ... activation-scale copies here (element kb of a route's row)
    const uint8_t* gS;              // ... (MXFP4) weight-scale copies here
    uint32_t offA[4], offB[kDmaB];  // ... plus these per-lane byte offsets
    uint32_t offX;                  // ... and this per-lane element offset
    uint32_t offS;                  // ... and this per-lane byte offset (MXFP4)
    int wave;                       // wave index (uniform)
    // fragment reads: lane's lower / upper half of weight tile 0 and route tile 0
    // (MXFP4: a_lo only, 16 bytes)
    int a_lo, a_hi, b_lo, b_hi;
    int x_off;                      // byte offset of the lane's route-tile-0 scale in a stage
    int na;                         // route tiles of this wave holding a route (uniform; the rest is padding)
    int a_step[4];                  // byte offsets of weight tiles 1..3 from tile 0 (constants)
    int s_off[4];                   // (MXFP4) byte offset of the lane's scale word in weight tile j
};


// A 16-byte global->LDS copy with a nontemporal load (data read once).
__device__ __forceinline__ void copy16_to_lds_nt(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :: "s"(lds), "v"(src) : "memory", "m0");
}

// Copy modes of the K loop's stage copies: plain; the activation tile and its
// scales at device scope (the producer); the FP8 weight tiles by nontemporal
// loads (read once per forward).
constexpr int kCopyPlain = 0, kCopyCoherent = 1, kCopyWeightsNt = 2;

// Issue the copies of K block kb into stage buffer st in copy mode kCopy.
template <bool kMx, int kCopy = kCopyPlain>
__device__ __forceinline__ void issue_stage(const Loop& L, uint8_t* st, int kb) {
    constexpr bool kCoh = kCopy == kCopyCoherent;
    using F = Fmt<kMx>;
    const uint8_t* gA = L.gA + (size_t)kb * F::kRowBytes;
    const uint8_t* gB = L.gB + (size_t)kb * 128;
    // (the destinations are wave-uniform; readfirstlane keeps them in scalar
    // registers for M0 whatever the compiler proves)
    const uint32_t base = lds_addr(st);
    auto dst = [&](uint32_t off) { return (uint32_t)__builtin_amdgcn_readfirstlane(base + off); };
    if constexpr (!kMx && kCopy == kCopyWeightsNt) {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) copy16_to_lds_nt(gA + L.offA[q], dst((L.wave * F::kDmaA + q) * 1024));
    } else {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) copy16_to_lds(gA + L.offA[q], dst((L.wave * F::kDmaA + q) * 1024));
    }
#pragma unroll
    for (int q = 0; q < kDmaB; ++q)
        copy16_to_lds<kCoh>(gB + L.offB[q], dst(F::kBOff + (L.wave * kDmaB + q) * 1024));
    // scales of routes 16 wave .. +16 (lanes 16..63 repeat lanes 0..15)
    copy4_to_lds<kCoh>(L.gX + L.offX + kb, dst(F::kXOff + L.wave * 256));
    // (MXFP4) the four scale bytes of K block kb of weight rows 32 wave ..
    // +32 (lanes 32..63 repeat lanes 0..31)
    if constexpr (kMx) copy4_to_lds(L.gS + L.offS + 4 * kb, dst(F::kAB + L.wave * 256));
}

// One K block on one wave: 4 weight tiles x 4 route tiles.  The raw block
// products of the previous K block (blk, with per-tile scales sw_p[j] *
// xr_p[m]) are promoted into acc just before the MFMA that overwrites them,
// so no promotion waits on the MFMA that has just been issued; this block's
// scales are handed back in sw_p / xr_p for the next call (before the first
// block, blk and the scales are zero, so that promotion adds zeros).  With
// MXFP4 weights the MFMA applies the weights' E8M0 scales itself and the
// promotion carries the activation scale alone.
// NA: only the wave's first NA route tiles hold routes (the others are
// padding rows, whose outputs are dropped): their fragments, MFMAs and
// promotions are left out, and each accumulator of the others sees the
// same operations in the same order.
template <bool kMx, int NA = 4>
__device__ __forceinline__ void block_mma(v4f acc[16], v4f blk[16], float sw_p[4], float xr_p[4], const Loop& L,
                                          const uint8_t* st, const float sw[4]) {
    if constexpr (NA == 0) return;
    v8i B[4];
    float xr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        xr[m] = 0.0f;
        if (m < NA) {   // (a constant once unrolled)
            B[m] = frag(st + L.b_lo + m * 2048, st + L.b_hi + m * 2048);
            xr[m] = *reinterpret_cast<const float*>(st + L.x_off + m * 256);
        }
    }
    if constexpr (kMx) {
        uint4 A[4];
        int sa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            A[j] = *reinterpret_cast<const uint4*>(st + L.a_lo + L.a_step[j]);
            sa[j] = st[L.s_off[j]];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if ((t & 3) >= NA) continue;
            const float sc = xr_p[t & 3];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(blk[t][v], sc, acc[t][v]);
            blk[t] = mfma_16x16x128_fp4_e4m3(A[t >> 2], B[t & 3], sa[t >> 2], v4f{0.0f, 0.0f, 0.0f, 0.0f});
        }
    } else {
        v8i A[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) A[j] = frag(st + L.a_lo + L.a_step[j], st + L.a_hi + L.a_step[j]);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if ((t & 3) >= NA) continue;
            const float sc = sw_p[t >> 2] * xr_p[t & 3];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(blk[t][v], sc, acc[t][v]);
            blk[t] = mfma_16x16x128_e4m3(A[t >> 2], B[t & 3], v4f{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sw_p[j] = sw[j];
        xr_p[j] = xr[j];
    }
}

// The whole K loop: KB blocks through three stage buffers, one barrier per
// block.  Step kb waits until this wave's copies of block kb have landed
// (block kb + 1 may stay in flight), and the barrier both makes every wave's
// copies of block kb visible and certifies that every wave has finished
// reading block kb - 1; only then are the copies of block kb + 2 issued, into
// kb - 1's buffer, so two blocks are in flight while block kb is multiplied.
// sw_of(kb, sw) fills the wave's four weight-tile scales of block kb (FP8
// weights).  The copies of blocks 0 and 1 (into buffers 0 and 1) are issued
// by the caller, possibly long before (issue_first).
template <bool kMx, int kCopy = kCopyPlain>
__device__ __forceinline__ void issue_first(const Loop& L, int KB, uint8_t* stages) {
    issue_stage<kMx, kCopy>(L, stages, 0);
    if (KB > 1) issue_stage<kMx, kCopy>(L, stages + Fmt<kMx>::kStage, 1);
}

// after_first() runs once, right after the first barrier: every wave has
// then finished whatever it did before the loop.
// Ring run-on (run_on, KB >= 2): the ring does not stop at the tile's end.
// At step KB - 2 (when this tile's copies are all issued) retarget(L) points
// L's copies at the next tile (its fragment geometry stays), the last two
// steps issue that tile's K blocks 0 and 1, the last step waits only for
// its own block, and the loop returns without a final barrier (the next
// tile's first barrier certifies that every wave has finished reading this
// tile's buffers before they are written again).  Block 0 sits in buffer
// rd0; the return value is the buffer of the next tile's block 0.
struct NoRetarget {
    __device__ void operator()(Loop&) const {}
};
template <bool kMx, int kCopy, int NA, typename SwOf, typename AfterFirst, typename Retarget>
__device__ __forceinline__ int k_loop_na(v4f acc[16], Loop& L, int KB, uint8_t* stages, SwOf sw_of,
                                         AfterFirst after_first, int rd0, bool run_on, Retarget retarget) {
    using F = Fmt<kMx>;
    float sw[4] = {1.0f, 1.0f, 1.0f, 1.0f}, sw_p[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xr_p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f blk[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) blk[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    run_on = run_on && KB >= 2;
    int rd = rd0;   // stage buffer of block kb
    for (int kb = 0; kb < KB; ++kb) {
        if (kb + 1 < KB || run_on) __builtin_amdgcn_s_waitcnt(vm_wait(F::kVmem));
        else __builtin_amdgcn_s_waitcnt(vm_wait(0));
        block_barrier();
        uint8_t* const wr = stages + (rd == 0 ? 2 : rd - 1) * F::kStage;
        if (kb + 2 < KB) {
            issue_stage<kMx, kCopy>(L, wr, kb + 2);
        } else if (run_on) {
            if (kb + 2 == KB) retarget(L);
            issue_stage<kMx, kCopy>(L, wr, kb + 2 - KB);
        }
        if (kb == 0) after_first();
        if constexpr (!kMx) sw_of(kb, sw);
        block_mma<kMx, NA>(acc, blk, sw_p, xr_p, L, stages + rd * F::kStage, sw);
        rd = rd == 2 ? 0 : rd + 1;
    }
    if (!run_on) block_barrier();   // every wave is done with the stage buffers
#pragma unroll
    for (int t = 0; t < 16; ++t) {   // promotion of the last block
        const float sc = kMx ? xr_p[t & 3] : sw_p[t >> 2] * xr_p[t & 3];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = fmaf(blk[t][v], sc, acc[t][v]);
    }
    return rd;
}

// The K loop for this wave's count of route tiles holding routes (L.na,
// wave-uniform; every instance waits, copies and meets the barriers alike):
// all four (one to four), or none; with kHalf also the first two (one or
// two).  The down kernel has the register room for two instances only.
template <bool kMx, int kCopy, bool kHalf, typename SwOf, typename AfterFirst, typename Retarget = NoRetarget>
__device__ __forceinline__ int k_loop(v4f acc[16], Loop& L, int KB, uint8_t* stages, SwOf sw_of,
                                      AfterFirst after_first, int rd0 = 0, bool run_on = false,
                                      Retarget retarget = Retarget{}) {
    if (L.na > (kHalf ? 2 : 0))
        return k_loop_na<kMx, kCopy, 4>(acc, L, KB, stages, sw_of, after_first, rd0, run_on, retarget);
    if (kHalf && L.na > 0)
        return k_loop_na<kMx, kCopy, 2>(acc, L, KB, stages, sw_of, after_first, rd0, run_on, retarget);
    return k_loop_na<kMx, kCopy, 0>(acc, L, KB, stages, sw_of, after_first, rd0, run_on, retarget);
}

// Roles of the 8 waves: wn (0..3) picks the weight rows of the tile, wr
// (0, 1) its 64-route half.  Waves w and w + 4 share a SIMD, so each SIMD
// holds one wave of each half: a tile whose second half is padding (an
// expert's last M-tile, every M-tile of a cold expert) then halves every
// SIMD's MFMA work instead of leaving two SIMDs with all of it.
__device__ __forceinline__ int route_half(int wave) { return wave >> 2; }
__device__ __forceinline__ int row_group(int wave) { return wave & 3; }
// Route tiles (of 16) of half wr that hold a route of a tile with `rows` routes.
__device__ __forceinline__ int route_tiles(int rows, int wr) {
    return __builtin_amdgcn_readfirstlane(min(4, max(0, (rows - 64 * wr + 15) >> 4)));
}

// (MXFP4) Slot of 16-byte chunk g of weight row r in a 64-byte LDS row is
// g ^ mx_swz(r): every 8 consecutive rows of one chunk fill the 8 16-byte
// slots of a 128-byte window, and rows 16 q .. 16 q + 15 fill those of a
// 256-byte window, so the A fragment reads (lane l: row l % 16, chunk l / 16)
// are free of bank conflicts for 8- or 16-lane service.  The activation rows
// of the MXFP4 kernels hold chunk p ^ swz(r) in slot p, so the B fragment
// reads (chunks g and g + 4) are free of conflicts too.
__device__ __forceinline__ int mx_swz(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }

// Fragment read offsets of this lane: row col of a 16-row tile, K group kg;
// weight tile j starts at LDS row a_row0 + a_rows[j], route tile 0 at row
// b_row0 (both multiples of 16).
template <bool kMx>
__device__ __forceinline__ void lane_geometry(Loop& L, int lane, int a_row0, const int (&a_rows)[4], int b_row0) {
    using F = Fmt<kMx>;
    const int col = lane & 15, kg = lane >> 4;
    if constexpr (kMx) {
        L.a_lo = (a_row0 + col) * 64 + (kg ^ mx_swz(col)) * 16;
        L.a_hi = L.a_lo;
        const int lo = kg ^ swz(col);   // chunks kg and kg + 4 of the route row
        L.b_lo = F::kBOff + (b_row0 + col) * 128 + lo * 16;
        L.b_hi = F::kBOff + (b_row0 + col) * 128 + (lo ^ 4) * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = a_row0 + a_rows[j] + col;
            L.a_step[j] = a_rows[j] * 64;
            L.s_off[j] = F::kAB + (r >> 5) * 256 + (r & 31) * 4 + kg;
        }
    } else {
        const int lo = lo_slot(col, kg);
        L.a_lo = (a_row0 + col) * 128 + lo * 16;
        L.a_hi = (a_row0 + col) * 128 + (lo ^ 4) * 16;
        L.b_lo = F::kBOff + (b_row0 + col) * 128 + lo * 16;
        L.b_hi = F::kBOff + (b_row0 + col) * 128 + (lo ^ 4) * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) L.a_step[j] = a_rows[j] * 128;
    }
    L.x_off = F::kXOff + (b_row0 / 16) * 256 + col * 4;
}

// Global byte offset, within a route's 128-byte K block, of the 16-byte
// chunk that lane slot p of route row r copies.
template <bool kMx>
__device__ __forceinline__ int act_chunk(int r, int p) {
    return (kMx ? (p ^ swz(r)) : chunk_of(r, p)) * 16;
}

// Both kernels are persistent: one workgroup per CU walks the tiles of its
// XCD's contiguous share (tile t of share x goes to workgroup x + 8 c with
// c = t mod (grid / 8)), so an expert's M-tiles still meet in one L2.  The
// next tile's token list and weight scales are requested at the start of the
// current tile's K loop, and the copies of its first two K blocks are issued
// before the current tile's epilogue, which then runs in their shadow.
struct TileSpan {
    int next, end, step;   // tile walk of this workgroup
};

__device__ __forceinline__ TileSpan tile_span(int n_tiles) {
    const int per_x = gridDim.x / 8, x = blockIdx.x % 8, c = blockIdx.x / 8;
    const int P = (n_tiles + 7) / 8;
    return TileSpan{x * P + c, min(n_tiles, (x + 1) * P), per_x};
}

struct TileInfo {
    int mt, sub;   // M-tile and column group (gate/up) or row tile (down)
    int e, beg, rows;
};

__device__ __forceinline__ TileInfo decode_tile(const TileMeta& meta, int E, int per_mt, int T) {
    TileInfo t;
    t.mt = T / per_mt;
    t.sub = T - t.mt * per_mt;
    t.e = __builtin_amdgcn_readfirstlane(tile_expert(meta.mtile_off, E, t.mt));
    t.beg = __builtin_amdgcn_readfirstlane(meta.offsets[t.e] + (t.mt - meta.mtile_off[t.e]) * kBM);
    t.rows = __builtin_amdgcn_readfirstlane(min(kBM, meta.offsets[t.e + 1] - t.beg));
    return t;
}

}  // namespace

// ------------------------------------------------- producer synchronisation

// Every workgroup of the grid arrives once at the device-scope word *ctr;
// returns when all n have (false when the wait timed out, and then also for
// the rest of the forward through flag).  Each workgroup's stores have
// completed before it arrives.  What one workgroup hands to another across a
// barrier is stored and loaded at device scope, so no cache needs writing
// back or invalidating (an agent-scope fence does both to a whole XCD L2,
// which measured about 11 us per barrier here).
__device__ __forceinline__ bool grid_barrier(uint32_t* ctr, uint32_t n, uint32_t* err, int tid, int& flag) {
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!wait_count(ctr, n, err, kErrProducer)) flag = 1;
    }
    __syncthreads();
    return flag == 0;
}

// ----------------------------------------------------------------- gate/up

namespace {

// Loop state of a gate/up tile.
// rt: the tile's route ids by row (padding rows repeat the last route).
template <bool kMx>
__device__ __forceinline__ Loop gate_up_loop(const PrefillArgs& a, const TileInfo& t, const int* rt, int wave,
                                             int lane) {
    using F = Fmt<kMx>;
    const int h = a.h, i = a.i, KB = h / 128, N13 = 2 * i;
    const int wr = route_half(wave), wn = row_group(wave);
    const int hb = kMx ? h / 2 : h;   // weight row bytes
    Loop L;
    // gate rows 32 wn + {0, 16}, up rows 128 + 32 wn + {0, 16}
    lane_geometry<kMx>(L, lane, 32 * wn, {0, 16, 128, 144}, 64 * wr);
    L.wave = wave;
    L.na = route_tiles(t.rows, wr);
    L.gA = a.w13 + (size_t)t.e * N13 * hb;
    L.gB = a.xq;
    L.gX = a.xs;
    auto wrow = [&](int r) { return r < 128 ? t.sub * 128 + r : i + t.sub * 128 + (r - 128); };
    if constexpr (kMx) {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) {   // 16 rows of 64 bytes per copy
            const int r = (wave * F::kDmaA + q) * 16 + (lane >> 2);
            L.offA[q] = (uint32_t)(wrow(r) * hb + ((lane & 3) ^ mx_swz(r)) * 16);
        }
        L.gS = a.e13 + (size_t)t.e * N13 * (h / 32);
        L.offS = (uint32_t)(wrow(32 * wave + (lane & 31)) * (h / 32));
    } else {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) {   // 8 rows of 128 bytes per copy
            const int r = (wave * F::kDmaA + q) * 8 + (lane >> 3);
            L.offA[q] = (uint32_t)(wrow(r) * hb + chunk_of(r, lane & 7) * 16);
        }
    }
#pragma unroll
    for (int q = 0; q < kDmaB; ++q) {
        const int r = (wave * kDmaB + q) * 8 + (lane >> 3);
        L.offB[q] = (uint32_t)(rt[r] / a.k * h + act_chunk<kMx>(r, lane & 7));
    }
    L.offX = (uint32_t)(rt[16 * wave + (lane & 15)] / a.k * KB);
    return L;
}

// Epilogue of a gate/up tile: SiLU(gate) * up and the 1x128 requantisation
// of group t.sub.  Tile u = 4 j + m: weight tile j (gate j = 0, 1; up j = 2,
// 3), route tile m.  Lane: route 64 wr + 16 m + col; gate/up columns
// 32 wn + 16 j + 4 kg + v of the group.  SiLU uses the hardware exp2 and
// reciprocal (a few ulp from the correctly rounded quotient; the FP8 block
// sums feeding it carry far larger error).  The codes are staged in LDS
// (codes, rows of 144 bytes so the 4-byte writes of 16 routes hit distinct
// banks) and leave as whole 128-byte rows.  kCoh: the codes and scales go
// out with device-scope stores (the producer's down tiles read them in the
// same launch, possibly on another XCD).
template <bool kCoh>
__device__ __forceinline__ void gate_up_epilogue(const PrefillArgs& a, const TileInfo& t, v4f acc[16],
                                                 float (*amax_l)[kBM], uint8_t* codes, int tid) {
    const int i = a.i, IB = i / 128;
    const int wave = tid >> 6, lane = tid & 63, col = lane & 15, kg = lane >> 4;
    const int wr = route_half(wave), wn = row_group(wave);
    const int na = route_tiles(t.rows, wr);   // route tiles past it hold only padding rows (never stored)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m >= na) continue;
        float pm = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float gt = acc[4 * j + m][v], up = acc[4 * (j + 2) + m][v];
                const float val = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                acc[4 * j + m][v] = val;
                pm = fmaxf(pm, fabsf(val));
            }
        pm = xor16_max(pm);
        pm = xor32_max(pm);
        if (kg == 0) amax_l[wn][64 * wr + 16 * m + col] = pm;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m >= na) continue;
        const int r = 64 * wr + 16 * m + col;
        const float sc =
            fmaxf(fmaxf(amax_l[0][r], amax_l[1][r]), fmaxf(amax_l[2][r], amax_l[3][r])) / kE4M3Max;
        const float rc = sc != 0.0f ? __builtin_amdgcn_rcpf(sc) : 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v4f vv = acc[4 * j + m];
            *reinterpret_cast<uint32_t*>(codes + r * 144 + 32 * wn + 16 * j + 4 * kg) =
                sc == 0.0f ? 0u : quant4(vv[0], vv[1], vv[2], vv[3], sc, rc);
        }
        if (wn == 0 && kg == 0 && r < t.rows) {
            float* ds = a.a2s + (size_t)(t.beg + r) * IB + t.sub;
            if constexpr (kCoh) st_agent(ds, sc);
            else *ds = sc;
        }
    }
    __syncthreads();
    const int r = tid >> 2, c = (tid & 3) * 32;   // 4 threads per route row, 32 bytes each
    if (r < t.rows) {
        const uint4* src = reinterpret_cast<const uint4*>(codes + r * 144 + c);
        uint4* dst = reinterpret_cast<uint4*>(a.a2 + (size_t)(t.beg + r) * i + t.sub * 128 + c);
        if constexpr (kCoh) {
            const uint64_t* s64 = reinterpret_cast<const uint64_t*>(src);
            uint64_t* d64 = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
            for (int q = 0; q < 4; ++q) st_agent64(d64 + q, s64[q]);
        } else {
            dst[0] = src[0];
            dst[1] = src[1];
        }
    }
}

// The gate/up tiles of this workgroup's share.  kProd (the producer): the
// route lists, activation codes and scales (written earlier in the same
// launch) are read at device scope, the requantised codes and scales go out
// at device scope, and each finished tile counts itself in its M-tile's word
// of a.done.
template <bool kMx, bool kProd, bool kNt = false>
__device__ __forceinline__ void gate_up_tiles(const PrefillArgs& a, TileLds<kMx>& S) {
    constexpr int kCopy = kProd ? kCopyCoherent : kNt ? kCopyWeightsNt : kCopyPlain;
    using F = Fmt<kMx>;
    uint8_t* const stages = S.stages;
    TileMeta& meta = S.meta;

    const int h = a.h, i = a.i, E = a.E;
    const int KB = h / 128, IB = i / 128, N13 = 2 * i;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

    load_meta<kProd>(meta, a, tid);
    __syncthreads();
    TileSpan span = tile_span(meta.mtile_off[E] * IB);
    if (span.next >= span.end) return;

    TileInfo t = decode_tile(meta, E, IB, span.next);
    int par = 0;
    // padding rows repeat the tile's last route (their outputs are dropped)
    for (int r = tid; r < kBM; r += kThreads) S.rt[0][r] = ld_i32<kProd>(a.sorted + t.beg + min(r, t.rows - 1));
    if constexpr (!kMx) {
        for (int j = tid; j < KB; j += kThreads) {
            S.sw[0][j] = a.s13[((size_t)t.e * (N13 / 128) + t.sub) * KB + j];
            S.sw[0][kMaxKB + j] = a.s13[((size_t)t.e * (N13 / 128) + IB + t.sub) * KB + j];
        }
    }
    __syncthreads();
    Loop L = gate_up_loop<kMx>(a, t, S.rt[0], wave, lane);
    issue_first<kMx, kCopy>(L, KB, stages);

    for (;;) {
        span.next += span.step;
        const bool more = span.next < span.end;
        TileInfo tn = t;
        if (more) tn = decode_tile(meta, E, IB, span.next);
        // The next tile's route ids (waves 0, 1) and, for FP8 weights, gate /
        // up scales (waves 2, 3) are copied straight into the other parity's
        // LDS lists during this tile's K loop (once its first barrier shows
        // that no wave still reads them), and its last wait and barrier also
        // cover these copies.  No register receives them, so the tile loop
        // carries no load the compiler would wait for.
        auto next_lists = [&]() {
            if (!more) return;
            if (wave < 2) {
                const int r = 64 * wave + lane;
                copy4_to_lds<kProd>(a.sorted + tn.beg + min(r, tn.rows - 1), lds_addr(&S.rt[par ^ 1][64 * wave]));
            } else if (!kMx && wave < 4) {
                const int half = wave - 2;
                const float* src = a.s13 + ((size_t)tn.e * (N13 / 128) + half * IB + tn.sub) * KB;
                for (int c = 0; 64 * c < KB; ++c)
                    copy4_to_lds(src + min(64 * c + lane, KB - 1), lds_addr(&S.sw[par ^ 1][half * kMaxKB + 64 * c]));
            }
        };
        auto sw_of = [&](int kb, float sw[4]) {
            const float g = S.sw[par][kb], u = S.sw[par][kMaxKB + kb];
            sw[0] = g; sw[1] = g; sw[2] = u; sw[3] = u;
        };
        v4f acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        k_loop<kMx, kCopy, true>(acc, L, KB, stages, sw_of, next_lists);   // ends with every wave done with the stage buffers
        if (more) {
            L = gate_up_loop<kMx>(a, tn, S.rt[par ^ 1], wave, lane);
            issue_first<kMx, kCopy>(L, KB, stages);   // buffers 0 and 1; the epilogue stages codes in buffer 2
        }
        gate_up_epilogue<kProd>(a, t, acc, S.amax, stages + 2 * F::kStage, tid);
        if constexpr (kProd) {
            // every wave's stores of the tile have completed before it counts
            wait_vmem();
            __syncthreads();
            if (tid == 0) __hip_atomic_fetch_add(a.done + t.mt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (!more) break;
        t = tn;
        par ^= 1;
    }
}

}  // namespace

// kNt: the weight tiles copied with nontemporal loads.
template <bool kNt>
__global__ __launch_bounds__(kThreads, 1) void prefill_gate_up_kernel(PrefillArgs a) {
    __shared__ TileLds<false> S;
    gate_up_tiles<false, false, kNt>(a, S);
}
__global__ __launch_bounds__(kThreads, 1) void prefill_gate_up_mx_kernel(PrefillArgs a) {
    __shared__ TileLds<true> S;
    gate_up_tiles<true, false>(a, S);
}

// -------------------------------------------------------------------- down

namespace {

template <bool kMx>
__device__ __forceinline__ Loop down_loop(const PrefillArgs& a, const TileInfo& t, int wave, int lane) {
    using F = Fmt<kMx>;
    const int h = a.h, i = a.i, IB = i / 128;
    const int wr = route_half(wave), wn = row_group(wave);
    const int ib = kMx ? i / 2 : i;   // weight row bytes
    Loop L;
    lane_geometry<kMx>(L, lane, 64 * wn, {0, 16, 32, 48}, 64 * wr);   // weight rows 64 wn + 16 j; route tiles 64 wr + 16 m
    L.wave = wave;
    L.na = route_tiles(t.rows, wr);
    L.gA = a.w2 + ((size_t)t.e * h + (size_t)t.sub * kBN) * ib;
    L.gB = a.a2 + (size_t)t.beg * i;
    L.gX = a.a2s + (size_t)t.beg * IB;
    if constexpr (kMx) {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) {
            const int r = (wave * F::kDmaA + q) * 16 + (lane >> 2);
            L.offA[q] = (uint32_t)(r * ib + ((lane & 3) ^ mx_swz(r)) * 16);
        }
        L.gS = a.e2 + ((size_t)t.e * h + (size_t)t.sub * kBN) * (i / 32);
        L.offS = (uint32_t)((32 * wave + (lane & 31)) * (i / 32));
    } else {
#pragma unroll
        for (int q = 0; q < F::kDmaA; ++q) {
            const int r = (wave * F::kDmaA + q) * 8 + (lane >> 3);
            L.offA[q] = (uint32_t)(r * ib + chunk_of(r, lane & 7) * 16);
        }
    }
#pragma unroll
    for (int q = 0; q < kDmaB; ++q) {
        const int r = (wave * kDmaB + q) * 8 + (lane >> 3);
        L.offB[q] = (uint32_t)(min(r, t.rows - 1) * i + act_chunk<kMx>(r, lane & 7));   // padding repeats the last route
    }
    L.offX = (uint32_t)(min(16 * wave + (lane & 15), t.rows - 1) * IB);
    return L;
}

// The down tiles of this workgroup's share.  kProd (the producer): a tile
// starts only once every gate/up tile of its M-tile has counted itself in
// (a.done), and reads their codes and scales at device scope; a wait that
// times out makes the workgroup give up the rest of its share.
template <bool kMx, bool kProd, bool kNt = false>
__device__ __forceinline__ void down_tiles(const PrefillArgs& a, TileLds<kMx>& S) {
    constexpr int kCopy = kProd ? kCopyCoherent : kNt ? kCopyWeightsNt : kCopyPlain;
    uint8_t* const stages = S.stages;
    TileMeta& meta = S.meta;

    const int h = a.h, i = a.i, E = a.E;
    const int IB = i / 128, NT = h / kBN;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int wr = route_half(wave), wn = row_group(wave);

    load_meta<kProd>(meta, a, tid);
    __syncthreads();
    TileSpan span = tile_span(meta.mtile_off[E] * NT);
    if (span.next >= span.end) return;

    // (producer) every wave waits until M-tile mt's IB gate/up tiles are done
    auto ready = [&](int mt) -> bool {
        if constexpr (kProd) {
            if (tid == 0 && S.flag == 0 && !wait_count(a.done + mt, (uint32_t)IB, a.err, kErrProducer)) S.flag = 1;
            __syncthreads();
            return S.flag == 0;
        } else {
            (void)mt;
            return true;
        }
    };

    TileInfo t = decode_tile(meta, E, NT, span.next);
    int par = 0;
    for (int r = tid; r < kBM; r += kThreads) S.rt[0][r] = ld_i32<kProd>(a.sorted + t.beg + min(r, t.rows - 1));
    if constexpr (!kMx) {   // j < 2 IB: scale blocks 2 sub and 2 sub + 1
        for (int j = tid; j < 2 * IB; j += kThreads) S.sw[0][j] = a.s2[((size_t)t.e * (h / 128) + 2 * t.sub) * IB + j];
    }
    __syncthreads();
    if (!ready(t.mt)) return;
    Loop L = down_loop<kMx>(a, t, wave, lane);
    issue_first<kMx, kCopy>(L, IB, stages);

    const int sblk = wn >> 1;
    int rd0 = 0;   // stage buffer of the tile's first K block
    for (;;) {
        span.next += span.step;
        const bool more = span.next < span.end;
        TileInfo tn = t;
        if (more) tn = decode_tile(meta, E, NT, span.next);
        // Outside the producer the ring runs on into the next tile (its
        // operands need no list from LDS), so that tile's first copies
        // travel during this tile's last K blocks instead of after them.
        constexpr bool kRunOn = !kProd;
        // the next tile's lists, copied straight into LDS as in the gate/up
        // kernel (the previous tile's epilogue read this parity's route list)
        auto next_lists = [&]() {
            if (!more) return;
            if (wave < 2) {
                const int r = 64 * wave + lane;
                copy4_to_lds<kProd>(a.sorted + tn.beg + min(r, tn.rows - 1), lds_addr(&S.rt[par ^ 1][64 * wave]));
            } else if (!kMx && 64 * (wave - 2) < 2 * IB) {
                const int c = wave - 2;
                const float* src = a.s2 + ((size_t)tn.e * (h / 128) + 2 * tn.sub) * IB;
                copy4_to_lds(src + min(64 * c + lane, 2 * IB - 1), lds_addr(&S.sw[par ^ 1][64 * c]));
            }
        };
        auto sw_of = [&](int kb, float sw[4]) {
            const float w = S.sw[par][sblk * IB + kb];
            sw[0] = w; sw[1] = w; sw[2] = w; sw[3] = w;
        };
        v4f acc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        auto retarget = [&](Loop& Lr) { Lr = down_loop<kMx>(a, tn, wave, lane); };
        rd0 = k_loop<kMx, kCopy, false>(acc, L, IB, stages, sw_of, next_lists, rd0, kRunOn && more, retarget);
        if (!(kRunOn && IB >= 2)) {
            rd0 = 0;
            if (more) {
                if (!ready(tn.mt)) return;   // no copy is in flight here
                L = down_loop<kMx>(a, tn, wave, lane);
                issue_first<kMx, kCopy>(L, IB, stages);
            }
        }
        // bf16 partial rows (round to nearest even) by route id; lane holds
        // output rows sub * 256 + 64 wn + 16 j + 4 kg + v of route
        // 64 wr + 16 m + col
        const int na = route_tiles(t.rows, wr);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m >= na) continue;
            const int row = 64 * wr + 16 * m + col;
            if (row >= t.rows) continue;
            const int p = S.rt[par][row];
            uint16_t* dst = a.y + (size_t)p * h + t.sub * kBN + 64 * wn + 4 * kg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f vv = acc[4 * j + m];
                *reinterpret_cast<uint2*>(dst + 16 * j) = make_uint2(bf16x2(vv[0], vv[1]), bf16x2(vv[2], vv[3]));
            }
        }
        if (!more) break;
        t = tn;
        par ^= 1;
    }
}

}  // namespace

template <bool kNt>
__global__ __launch_bounds__(kThreads, 1) void prefill_down_kernel(PrefillArgs a) {
    __shared__ TileLds<false> S;
    down_tiles<false, false, kNt>(a, S);
}
__global__ __launch_bounds__(kThreads, 1) void prefill_down_mx_kernel(PrefillArgs a) {
    __shared__ TileLds<true> S;
    down_tiles<true, false>(a, S);
}

// ---------------------------------------------------------------- producer

namespace {

// The whole layer but the route reducer in one launch (the producer of the
// Netra Kernel README's MoE prefill pair: routing, gate/up, SiLU and
// requantisation, down-partial and metadata in one code object; the
// reducer, combine_bf16_kernel, is the second).  One workgroup per CU, all
// resident at once:
//   1. every workgroup routes and quantises its chunk of tpw tokens and
//      counts the chunk's routes per expert into its row of hist;
//   2. grid barrier; each chunk sums the counts and scatters its routes in
//      route order (group_chunk_scatter; chunk 0 writes counts, offsets, the
//      active list and the M-tile numbering);
//   3. grid barrier; the gate/up tiles of the workgroup's share, each
//      counted in its M-tile's word of done once its codes are stored;
//   4. the down tiles of its share, each after its M-tile's count reaches
//      i/128.
// A workgroup reaches step 4 only after all its gate/up tiles, so every wait
// is for work that waits on nothing, and every wait is bounded in time (a
// timeout sets kErrProducer in the error word, the workgroup gives up its
// share, and the reducer writes NaN).  The last workgroup to finish clears
// the counters for the next forward.
template <bool kMx>
__device__ __forceinline__ void producer_tiles(const ProducerArgs& p) {
    __shared__ TileLds<kMx> S;
    const PrefillArgs& a = p.pa;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int M = p.M, E = a.E, k = a.k, h = a.h;
    const uint32_t G = gridDim.x;
    const int nchunks = (M + p.tpw - 1) / p.tpw;
    const int t0 = blockIdx.x * p.tpw, t1 = min(M, t0 + p.tpw);
    int* scr = reinterpret_cast<int*>(S.stages);   // the stage ring is free until step 3
    uint32_t* bar = p.sync + kSyncProdBar / 4;
    if (tid == 0) {
        S.flag = 0;
        S.last = 0;
    }
    for (int e = tid; e < 256; e += kThreads) scr[e] = 0;

    // 1. routing (four tokens per wave and pass) and quantisation (one row
    // per wave at a time): the loads of a wave's first four rows go out
    // first and the routing runs under them
    if (t0 < M) {
        constexpr int kNW = kThreads / kWave;
        uint4 u[4][kQuantBatch];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + wave + kNW * j;
            if (t < t1) act_quant_load(p.x + (size_t)t * h, h, 0, 0, 1, lane, u[j]);
        }
        for (int c = wave; t0 + 4 * c < t1; c += kNW) router_rows16(p.logits, t0 + 4 * c, t1, E, k, p.ids, p.tw, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + wave + kNW * j;
            if (t < t1)
                act_quant_finish<true>(p.x + (size_t)t * h, h, p.xq + (size_t)t * h, p.xs + (size_t)t * (h / 128), 0,
                                       1, lane, u[j]);
        }
        for (int t = t0 + wave + 4 * kNW; t < t1; t += kNW)
            act_quant_row<true>(p.x + (size_t)t * h, h, p.xq + (size_t)t * h, p.xs + (size_t)t * (h / 128), 0, 1, lane);
    }
    wait_vmem();
    __syncthreads();
    if (t0 < M) group_chunk_hist(p.ids, t0 * k, t1 * k, E, scr, tid, kThreads);
    __syncthreads();
    if ((int)blockIdx.x < nchunks && tid < E) st_i32<true>(p.hist + (size_t)blockIdx.x * E + tid, scr[tid]);
    bool ok = grid_barrier(bar, G, a.err, tid, S.flag);

    // 2. grouping
    if (ok && (int)blockIdx.x < nchunks) {
        const GroupOut o{p.counts, p.offsets, p.sorted, p.active, p.num_active, p.mtile_off, kBM};
        group_chunk_scatter<kThreads / 256, true, 32>(p.ids, E, nchunks, p.hist, blockIdx.x, t0 * k, t1 * k,
                                                      blockIdx.x == 0, o, scr, scr + 512, scr + 1024, tid);
    }
    ok = grid_barrier(bar + 1, G, a.err, tid, S.flag);

    // 3., 4. the GEMMs
    if (ok) gate_up_tiles<kMx, true>(a, S);
    __syncthreads();
    if (S.flag == 0) down_tiles<kMx, true>(a, S);

    // the last workgroup to finish clears the counters (all of them after a
    // timeout, else the M-tiles of this forward)
    wait_vmem();
    __syncthreads();
    if (tid == 0) S.last = __hip_atomic_fetch_add(p.sync + kSyncProdExit / 4, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) == G - 1;
    __syncthreads();
    if (S.last) {
        const bool timed_out = (ld_agent(a.err) & kErrProducer) != 0u;
        const int n = timed_out ? kProdMaxTiles : min(kProdMaxTiles, ld_agent(reinterpret_cast<const uint32_t*>(p.mtile_off) + E));
        for (int j = tid; j < n; j += kThreads) st_agent(a.done + j, 0u);
        if (tid == 0) {
            st_agent(bar, 0u);
            st_agent(bar + 1, 0u);
            st_agent(p.sync + kSyncProdExit / 4, 0u);
        }
    }
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void prefill_producer_kernel(ProducerArgs p) { producer_tiles<false>(p); }
__global__ __launch_bounds__(kThreads, 1) void prefill_producer_mx_kernel(ProducerArgs p) { producer_tiles<true>(p); }

int prefill_tile_m() { return kBM; }

bool prefill_supported(int M, int h, int i, int k) {
    const int64_t lim = (int64_t)1 << 31;   // 32-bit per-lane offsets
    return h % kBN == 0 && i % 128 == 0 && h <= 128 * kMaxKB && i <= 128 * kMaxKB && (int64_t)M * h < lim &&
           (int64_t)M * k * i < lim && (int64_t)M * (h / 128) < lim;
}

// One workgroup per CU (the grid must be a multiple of 8, one share per XCD).
static int persistent_grid() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static int cached[64] = {0};
    if (dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = std::max(8, cus / 8 * 8);
    }
    return cached[dev];
}

// mx: the weights are MXFP4 (w13 / w2 codes with e13 / e2 scales), else FP8
// (with s13 / s2).
// Every M-tile needs a counter word: at most ceil(R / 128) + E tiles.
bool producer_supported(int M, int h, int i, int E, int k) {
    const int64_t R = (int64_t)M * k;
    return prefill_supported(M, h, i, k) && (R + kBM - 1) / kBM + E <= kProdMaxTiles;
}

// One workgroup per CU, and all of them resident at once (checked against
// the kernel's occupancy, cached per device).
hipError_t launch_prefill_producer(const ProducerArgs& p, bool mx, hipStream_t stream) {
    const int g = persistent_grid();
    if (g <= 0 || g > kProdMaxGrid) return hipErrorInvalidDevice;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static int fits[2][64] = {{0}};   // 0: not known, 1: fits, -1: does not
    int& f = fits[mx ? 1 : 0][dev];
    if (f == 0) {
        int cu = 0, nb = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        const hipError_t e = mx ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, prefill_producer_mx_kernel, kThreads, 0)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, prefill_producer_kernel, kThreads, 0);
        if (e != hipSuccess) return hipErrorInvalidConfiguration;
        f = cu * nb >= g ? 1 : -1;
    }
    if (f < 0) return hipErrorInvalidConfiguration;
    ProducerArgs q = p;
    q.tpw = std::max(4, (p.M + g - 1) / g);   // at most g routing chunks
    if (mx) launch(prefill_producer_mx_kernel, dim3(g), dim3(kThreads), 0, stream, q);
    else launch(prefill_producer_kernel, dim3(g), dim3(kThreads), 0, stream, q);
    return hipGetLastError();
}

hipError_t launch_prefill_gate_up(const PrefillArgs& a, bool mx, hipStream_t stream) {
    const int g = persistent_grid();
    if (g <= 0) return hipErrorInvalidDevice;
    if (mx) launch(prefill_gate_up_mx_kernel, dim3(g), dim3(kThreads), 0, stream, a);
    else if (a.weights_nt) launch(prefill_gate_up_kernel<true>, dim3(g), dim3(kThreads), 0, stream, a);
    else launch(prefill_gate_up_kernel<false>, dim3(g), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_down(const PrefillArgs& a, bool mx, hipStream_t stream) {
    const int g = persistent_grid();
    if (g <= 0) return hipErrorInvalidDevice;
    if (mx) launch(prefill_down_mx_kernel, dim3(g), dim3(kThreads), 0, stream, a);
    else if (a.weights_nt) launch(prefill_down_kernel<true>, dim3(g), dim3(kThreads), 0, stream, a);
    else launch(prefill_down_kernel<false>, dim3(g), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moe
