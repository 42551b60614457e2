// probe.hip -- measurement kernels that frame the layer's numbers: an empty
// kernel (what a launch costs by itself inside a graph) and a plain
// streaming read (how fast one launch can pull a given number of bytes from
// HBM).  Neither is on the forward path.
#include "device.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void probe_empty_kernel() {}

// Every thread reads 16-byte words in a grid-stride loop with four loads in
// flight, folds them with xor, and one lane per workgroup writes the fold so
// the loads cannot be dropped.  `words` 16-byte words at `src`.
__global__ __launch_bounds__(256) void probe_read_kernel(const v4i* __restrict__ src, size_t words,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
    v4i acc = {0, 0, 0, 0};
    for (; j + 3 * stride < words; j += 4 * stride) {
        const v4i a = __builtin_nontemporal_load(src + j);
        const v4i b = __builtin_nontemporal_load(src + j + stride);
        const v4i c = __builtin_nontemporal_load(src + j + 2 * stride);
        const v4i d = __builtin_nontemporal_load(src + j + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; j < words; j += stride) acc ^= __builtin_nontemporal_load(src + j);
    uint32_t f = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
    for (int o = 32; o > 0; o >>= 1) f ^= (uint32_t)__shfl_xor((int)f, o);
    const uint32_t acc_out = f;
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc_out;
}

hipError_t launch_probe_empty(int grid, hipStream_t stream) {
    hipLaunchKernelGGL(probe_empty_kernel, dim3(grid), dim3(256), 0, stream);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const v4i*>(src),
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
