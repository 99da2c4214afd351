// Split-KV decode, second pass: log-sum-exp combination of the chunk states.
//
// "GPT-OSS on day 0" (Perplexity), Kernels for GPT-OSS / Sink attention,
// parallelises attention along the KV sequence but does not say how the
// blocks' results are combined.  The combination used here is the one that
// makes the result independent of the split: with M = max_c m_c and
// w_c = e^(m_c - M), out = sum_c w_c acc_c / sum_c w_c d_c and
// lse = M + ln sum_c w_c d_c.  The sink already sits in the state of the block
// that holds the sequence's first key.
//
// One wave per (sequence, query head), lane = output dimension.  Up to 64 blocks
// are combined from one round trip: lane c reads block c's m and d, every lane
// reads its dimension of each block's accumulator (all of those loads issued
// before any is used, in groups of kGroup rows), and the maximum and the weighted
// scale sum are wave reductions.  Past 64 blocks, further passes of 64 fold in
// with the usual rescale of the running sums.  The first pass's loads go out
// before the sequence's block count is known (slots clamped to the buffer and
// masked afterwards).
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kGroup = 16;  // accumulator rows per group of loads

// Butterfly over the wave: lane pairs 1 and 2 apart (quad permutes), then 4 and 8
// (row half-mirror, row mirror), 16 (swizzle) and 32 (lane swap); every lane ends
// with the reduction of all 64.
template <bool kMax>
__device__ __forceinline__ float wave_reduce(float x) {
    auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true)));
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true)));
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true)));
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true)));
    x = op(x, xor16(x));
    return kMax ? max_xor32(x) : sum_xor32(x);
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// cu_k == nullptr: every one of the plan.max_chunks slots of each row holds a state
// (rows of a split prefill, [rows, Hq, slots]).  Otherwise the blocks of sequence b
// under `plan`, in the plan's slot layout.
template <bool kBf16>
__global__ __launch_bounds__(64 * kWavesPerBlock) void merge_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_d,
    const float* __restrict__ part_acc, const int32_t* __restrict__ cu_k, DecodePlan plan,
    int batch, int hq, void* __restrict__ out, float* __restrict__ lse) {
    // (the wave index is uniform: keep it, and every index derived from it, scalar)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
    const int pair = blockIdx.x * kWavesPerBlock + wave;
    if (pair >= batch * hq) return;  // no workgroup barrier below
    const int b = pair / hq, h = pair - b * hq;
    const int nc = plan.max_chunks;
    const SlotLayout lay = cu_k != nullptr ? plan_slots(plan, hq) : head_major_slots(hq, nc);
    const int64_t s0 = b * lay.seq + h * lay.head;  // slot of block 0
    auto slot = [&](int c) { return s0 + (int64_t)min(c, nc - 1) * lay.block; };

    // first pass, before the block count is known: m and d of blocks 0..63 (lane = block)
    // and the first group of accumulator rows
    float m_ld = part_m[slot(lane)];
    float d_ld = part_d[slot(lane)];
    float a[4][kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) a[0][u] = part_acc[slot(u) * kD + lane];
    __builtin_amdgcn_sched_barrier(0);

    int nch = nc;
    if (cu_k != nullptr) {
        const int k_lo = cu_k[b], k_hi = cu_k[b + 1];
        if (plan.chunk > 0) {
            nch = ceil_div(max(k_hi - k_lo, 0), plan.chunk);
        } else {
            const int base = cu_k[0], total = cu_k[batch] - base;
            const int extra = balanced_extra_blocks(total, batch, plan);
            nch = balanced_first_block(k_hi - base, b + 1, total, extra) -
                  balanced_first_block(k_lo - base, b, total, extra);
        }
        nch = max(1, min(nch, nc));
    }

    float big = kNegInf, acc = 0.0f, den = 0.0f;
    for (int r0 = 0;;) {  // passes of up to 64 blocks
        const int nr = min(nch - r0, 64);
        const int groups = ceil_div(nr, kGroup);
        // the rest of this pass's accumulator rows, every load before any use
        if (r0 > 0) {
#pragma unroll
            for (int u = 0; u < kGroup; ++u) a[0][u] = part_acc[slot(r0 + u) * kD + lane];
        }
#pragma unroll
        for (int gi = 1; gi < 4; ++gi)
            if (gi < groups) {
#pragma unroll
                for (int u = 0; u < kGroup; ++u)
                    a[gi][u] = part_acc[slot(r0 + gi * kGroup + u) * kD + lane];
            }
        const bool mine = lane < nr;
        const float ml = mine ? m_ld : kNegInf;
        const float rbig = wave_reduce<true>(ml);
        if (rbig != kNegInf) {  // (uniform) some block of the pass holds mass
            const float nb = fmaxf(big, rbig);
            if (big != kNegInf && nb != big) {
                const float sc = fast_exp2((big - nb) * kLog2e);
                acc *= sc;
                den *= sc;
            }
            big = nb;
            // weight 0 past the end and for empty blocks, whose slots may hold
            // anything there: select, do not multiply
            const float wl = ml == kNegInf ? 0.0f : fast_exp2((ml - big) * kLog2e);
            den += wave_reduce<false>(wl != 0.0f ? wl * d_ld : 0.0f);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi)
                if (gi < groups) {
#pragma unroll
                    for (int u = 0; u < kGroup; ++u) {
                        const float w = lane_value(wl, gi * kGroup + u);
                        acc += w != 0.0f ? w * a[gi][u] : 0.0f;
                    }
                }
        }
        r0 += 64;
        if (r0 >= nch) break;
        m_ld = part_m[slot(r0 + lane)];
        d_ld = part_d[slot(r0 + lane)];
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

hipError_t launch(bool out_bf16, const float* part_m, const float* part_d, const float* part_acc,
                  const int32_t* cu_k, const DecodePlan& plan, int batch, int hq, void* out,
                  float* lse, hipStream_t stream) {
    const int pairs = batch * hq;
    dim3 grid(ceil_div(pairs, kWavesPerBlock));
    if (out_bf16)
        hipLaunchKernelGGL((merge_kernel<true>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           part_m, part_d, part_acc, cu_k, plan, batch, hq, out, lse);
    else
        hipLaunchKernelGGL((merge_kernel<false>), grid, dim3(64 * kWavesPerBlock), 0, stream,
                           part_m, part_d, part_acc, cu_k, plan, batch, hq, out, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(bool out_bf16, const float* part_m, const float* part_d,
                        const float* part_acc, const int32_t* cu_k, int chunk, int max_chunks,
                        int batch, int hq, void* out, float* lse, hipStream_t stream) {
    const DecodePlan plan{chunk, 0, 0, max_chunks};
    return launch(out_bf16, part_m, part_d, part_acc, cu_k, plan, batch, hq, out, lse, stream);
}

hipError_t launch_merge_plan(bool out_bf16, const float* part_m, const float* part_d,
                             const float* part_acc, const int32_t* cu_k, const DecodePlan& plan,
                             int batch, int hq, void* out, float* lse, hipStream_t stream) {
    return launch(out_bf16, part_m, part_d, part_acc, cu_k, plan, batch, hq, out, lse, stream);
}

}  // namespace sa
