// Streaming-read yardstick: one pass over a device buffer with the nontemporal
// 16-byte loads that the split-KV decode uses for its K/V stream.  It is not a
// step of the attention method; it measures the practical read rate of the
// device's HBM, against which the HBM-bound kernels can be compared, and its XOR
// digest makes the pass checkable.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 4;  // 16-byte loads in flight per thread and iteration

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint16_t* __restrict__ p,
                                                              int64_t n16,
                                                              uint32_t* __restrict__ out) {
    __shared__ uint32_t part[kThreads / 64];
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n16; i += stride) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * kThreads;
            x[u] = j < n16 ? load_stream(p + 8 * j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    }
    // XOR over the wave, then over the workgroup's waves
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) acc ^= __shfl_xor(acc, off, 64);
    if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) t ^= part[w];
        out[blockIdx.x] = t;
    }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, int num_blocks, uint32_t* out,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(num_blocks), dim3(kThreads), 0, stream,
                       (const uint16_t*)buf, bytes / 16, out);
    return hipGetLastError();
}

}  // namespace sa
