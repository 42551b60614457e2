// fused_decode.h -- arguments and launcher of the one-kernel decode forward
// (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

struct FusedArgs {
    const uint16_t* x;
    const float* logits;
    const uint8_t* w13;
    const float* s13;
    const uint8_t* w2;
    const float* s2;
    uint16_t* out;
    int M, h, i, E, k;
    // routing and quantisation published by workgroup 0 (inspection)
    int32_t* ids;
    float* tw;
    uint8_t* xq;
    float* xs;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* num_active;
    // exchange buffers: 64-bit (value, forward tag) words
    uint64_t* v_ll;   // [M*k][i]       SiLU(gate) * up by route
    uint64_t* t_ll;   // [M*k][i/128][h] down block terms by route and K block
    // synchronisation words
    uint32_t* sync;
};

bool fused_supported(int M, int h, int i, int E, int k);
int fused_parts(int M, int i, int E, int k);
// Words of the v exchange buffer; t follows it, rounded up to 32 words.
inline size_t fused_v_words(int M, int i, int k) { return ((size_t)M * k * i + 31) & ~(size_t)31; }
size_t fused_lds_bytes(int M, int h, int i, int E, int k);
hipError_t launch_fused_decode(const FusedArgs& args, hipStream_t stream);

// Sync-word region at the start of every workspace, then the fused path's
// exchange region (fixed place, so no other path ever writes there).
constexpr size_t kSyncBytes = 32768;
constexpr size_t kSyncEpoch = 0;                // word: forwards run on this workspace
constexpr size_t kSyncExit = 256;               // word: workgroups finished in this forward
constexpr size_t kSyncErr = 512;                // word: sticky error (a wait timed out)
constexpr size_t kSyncArrive = 1024;            // word: routing workgroups counted in (grouping tail)
constexpr size_t kSyncProdBar = 1280;           // two words: the prefill producer's grid barriers
constexpr size_t kSyncProdExit = 1536;          // word: producer workgroups finished in this forward
constexpr size_t kSyncProdDone = 4096;          // words: gate/up tiles finished, per M-tile (producer)
constexpr int kProdMaxTiles = (int)((kSyncBytes - kSyncProdDone) / 4);
// Bits of the sticky error word: a wait of the one-kernel decode path, or of
// the prefill producer, timed out.
constexpr uint32_t kErrFused = 1u;
constexpr uint32_t kErrProducer = 2u;
constexpr size_t kLLBytes = (size_t)8 << 20;    // v_ll, then t_ll
constexpr size_t kLLOffset = kSyncBytes;
constexpr size_t kWorkspaceHead = kSyncBytes + kLLBytes;   // zero-initialised part
hipError_t launch_zero_words(uint32_t* p, size_t words, hipStream_t stream);

}  // namespace moe
