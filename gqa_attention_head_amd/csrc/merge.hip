// Split-KV decode, second pass: log-sum-exp combination of the chunk states.
//
// "GPT-OSS on day 0" (Perplexity), Kernels for GPT-OSS / Sink attention,
// parallelises attention along the KV sequence but does not say how the
// blocks' results are combined.  The combination used here is the one that
// makes the result independent of the split: with M = max_c m_c and
// w_c = e^(m_c - M), out = sum_c w_c acc_c / sum_c w_c d_c and
// lse = M + ln sum_c w_c d_c.  The sink already sits in chunk 0's state.
//
// One wave per (sequence, query head); lane = output dimension (head_dim 64).
// The wave first finds M (lanes stride over the chunks), then each lane
// computes the weight of one chunk and the lanes sweep the chunks' rows for
// their own dimension, the weights broadcast across the wave.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <bool kBf16>
__global__ __launch_bounds__(64 * kWavesPerBlock) void merge_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_d,
    const float* __restrict__ part_acc, const int32_t* __restrict__ cu_k, int chunk,
    int max_chunks, int batch, int hq, void* __restrict__ out, float* __restrict__ lse) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int pair = blockIdx.x * kWavesPerBlock + wave;
    if (pair >= batch * hq) return;  // no workgroup barrier below
    const int b = pair / hq;
    const int len = cu_k[b + 1] - cu_k[b];
    const int nch = min(max_chunks, max(1, ceil_div(len, chunk)));
    const int64_t base = (int64_t)pair * max_chunks;

    float big = kNegInf;
    for (int c = lane; c < nch; c += 64) big = fmaxf(big, part_m[base + c]);
    big = wave_max(big);

    float acc = 0.0f, den = 0.0f;
    if (big != kNegInf) {
        for (int c0 = 0; c0 < nch; c0 += 64) {
            // lane j of the group holds chunk c0 + j's weight
            const int c = c0 + lane;
            float w = 0.0f, dw = 0.0f;
            if (c < nch) {
                const float mc = part_m[base + c];
                w = (mc == kNegInf) ? 0.0f : fast_exp2((mc - big) * kLog2e);
                dw = w * part_d[base + c];
            }
            den += wave_sum(dw);
            const int n = min(64, nch - c0);
            // lane = output dimension; eight chunk rows in flight at a time
            for (int j0 = 0; j0 < n; j0 += 8) {
                float vals[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    vals[u] = (j0 + u < n) ? part_acc[(base + c0 + j0 + u) * kD + lane] : 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += __shfl(w, j0 + u) * vals[u];
            }
        }
    }
    const bool empty = (big == kNegInf) || !(den > 0.0f);
    const float o = empty ? 0.0f : acc / den;
    const int64_t orow = (int64_t)pair * kD + lane;
    if (kBf16)
        reinterpret_cast<uint16_t*>(out)[orow] = f32_to_bf16_bits(o);
    else
        reinterpret_cast<float*>(out)[orow] = o;
    if (lse != nullptr && lane == 0) lse[pair] = empty ? kNegInf : big + fast_log2(den) * kLn2;
}

}  // namespace

hipError_t launch_merge(bool out_bf16, const float* part_m, const float* part_d,
                        const float* part_acc, const int32_t* cu_k, int chunk, int max_chunks,
                        int batch, int hq, void* out, float* lse, hipStream_t stream) {
    const int pairs = batch * hq;
    dim3 grid(ceil_div(pairs, kWavesPerBlock));
    if (out_bf16)
        hipLaunchKernelGGL((merge_kernel<true>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           part_m, part_d, part_acc, cu_k, chunk, max_chunks, batch, hq, out, lse);
    else
        hipLaunchKernelGGL((merge_kernel<false>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           part_m, part_d, part_acc, cu_k, chunk, max_chunks, batch, hq, out, lse);
    return hipGetLastError();
}

}  // namespace sa
