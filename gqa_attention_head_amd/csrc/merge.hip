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
// The chunk states are read in groups of kGroup chunks, every load of a group
// issued before any is used (a single round trip for up to kGroup chunks); a
// later group, if any, folds in with the usual rescale of the running sums.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kGroup = 16;  // chunk states loaded per round trip

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
    const int64_t base = (int64_t)pair * max_chunks;

    // The first group's loads do not wait for the sequence length: they read
    // slots clamped to the buffer's last one and are masked once nch is known.
    const int k_lo = (cu_k != nullptr) ? cu_k[b] : 0;
    const int k_hi = (cu_k != nullptr) ? cu_k[b + 1] : 0;
    float m_ld, d_ld, av[kGroup];
    auto load_group = [&](int c0) {
        // lane u < kGroup: chunk c0 + u's m and d; every lane: its dimension of
        // the kGroup accumulators
        const int cl = min(c0 + lane % kGroup, max_chunks - 1);
        m_ld = part_m[base + cl];
        d_ld = part_d[base + cl];
#pragma unroll
        for (int u = 0; u < kGroup; ++u)
            av[u] = part_acc[(base + min(c0 + u, max_chunks - 1)) * kD + lane];
    };
    load_group(0);
    __builtin_amdgcn_sched_barrier(0);
    // without sequence lengths every slot holds a state (rows of a split prefill)
    const int nch = (cu_k != nullptr) ? min(max_chunks, max(1, ceil_div(k_hi - k_lo, chunk)))
                                      : max_chunks;

    float big = kNegInf, acc = 0.0f, den = 0.0f;
    for (int c0 = 0;;) {
        const bool mine = lane < kGroup && c0 + lane < nch;
        const float ml = mine ? m_ld : kNegInf;
        const float nbig = fmaxf(big, wave_max(ml));
        if (nbig != kNegInf) {  // (uniform) otherwise nothing finite yet
            if (nbig != big) {
                const float scale = (big == kNegInf) ? 0.0f : fast_exp2((big - nbig) * kLog2e);
                acc *= scale;
                den *= scale;
                big = nbig;
            }
            const float wl = (ml == kNegInf) ? 0.0f : fast_exp2((ml - big) * kLog2e);
            den += wave_sum(mine ? wl * d_ld : 0.0f);
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                // chunk c0 + u's weight, from lane u (0 for chunks past the end,
                // whose slots may hold anything: select, do not multiply)
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
                acc += (w != 0.0f) ? w * av[u] : 0.0f;
            }
        }
        c0 += kGroup;
        if (c0 >= nch) break;
        load_group(c0);
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
