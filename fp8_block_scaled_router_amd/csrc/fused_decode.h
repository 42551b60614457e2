// fused_decode.h -- arguments and launcher of the one-kernel small-batch
// forward (internal to the library).
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
    int umax;  // min(E, M*k): bound on the number of experts with routes
    // intermediates published / exchanged through the workspace
    int32_t* ids;
    float* tw;
    uint8_t* xq;
    float* xs;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* num_active;
    float* g;
    uint8_t* a2;
    float* a2s;
    float* y;
    // synchronisation words (zero between forwards)
    uint32_t* gate_tix;  // [umax][i/128]
    uint32_t* done;      // [umax]
    uint32_t* comb_tix;  // [M][h/64]
    uint32_t* exit_cnt;  // [1]
    uint32_t* err;       // [1], sticky: set when a wait timed out
};

bool fused_supported(int M, int h, int i, int E, int k);
size_t fused_lds_bytes(int M, int h, int i, int E, int k);
hipError_t launch_fused_decode(const FusedArgs& args, hipStream_t stream);

// Sync-word region at the start of every workspace.
constexpr size_t kSyncBytes = 32768;
constexpr size_t kSyncGateTix = 0;              // 4096 words
constexpr size_t kSyncDone = 16384;             // 256 words
constexpr size_t kSyncCombTix = 17408;          // 2048 words
constexpr size_t kSyncExit = 25600;             // 1 word
constexpr size_t kSyncErr = 25856;              // 1 word
hipError_t launch_zero_words(uint32_t* p, size_t words, hipStream_t stream);

}  // namespace moe
