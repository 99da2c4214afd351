// Top-K-then-softmax expert routing, bf16 logits (gfx950).
//
// "GPT-OSS on day 0" (Perplexity), MoE section: the gpt-oss router takes the
// softmax over the K selected experts only, and the expert weights are bf16.
// For every token: the K experts with the largest logits (larger first, equal
// logits by lower expert index) and the softmax of those K logits, computed in
// float32 and rounded to bf16.
//
// Layout: a token's E logits are spread over E/32 lanes (one lane for E < 32),
// each holding 32 (or E) logits, so a wave covers a contiguous run of whole token
// rows.  The wave reads that run with nontemporal 16-byte loads, each instruction
// one contiguous 1 KB, into its own LDS slice, and every lane then reads its
// logits from there.  Each logit becomes one 32-bit key whose
// unsigned order is the ranking: the high half maps the bf16 value to an
// order-preserving code (-0 folded onto +0; two codes per word with packed 16-bit
// arithmetic), the low half holds 31 - (position in the lane), so a larger key is
// a larger logit or, on a tie, a lower expert.  Each lane inserts its keys into a
// descending list of its KP largest (one max and KP - 1 three-way medians per
// key), then turns the low halves into 0xFFFF - expert; round r takes the largest
// head across the token's lanes (DPP and lane-swap maxima, no LDS), and the lane
// that held it moves on to its next key.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

// value of a key's order code (high half): 0x8000 + m for +m, 0x8000 - m for -m
__device__ __forceinline__ float code_value(uint32_t code) {
    const uint32_t bits = (code >= 0x8000u) ? (code - 0x8000u) : ((0x8000u - code) | 0x8000u);
    return bf16_bits_to_f32(static_cast<uint16_t>(bits));
}

// Maximum over each aligned group of kLanes lanes, left in every lane of the group:
// DPP swaps and mirrors inside a 16-lane row, then the cross-row lane swaps.
template <int kLanes>
__device__ __forceinline__ uint32_t group_max(uint32_t x) {
    auto dpp = [](uint32_t v, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, decltype(ctrl)::value, 0xF, 0xF, false);
    };
    if (kLanes >= 2) x = max(x, dpp(x, std::integral_constant<int, 0xB1>{}));   // quad_perm 1,0,3,2
    if (kLanes >= 4) x = max(x, dpp(x, std::integral_constant<int, 0x4E>{}));   // quad_perm 2,3,0,1
    if (kLanes >= 8) x = max(x, dpp(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    if (kLanes >= 16) x = max(x, dpp(x, std::integral_constant<int, 0x140>{})); // row_mirror
    if (kLanes >= 32)
        x = max(x, (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F));       // lane ^ 16
    if (kLanes >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);            // lane ^ 32
        x = max(r[0], r[1]);
    }
    return x;
}

constexpr int next_pow2(int k) { return k <= 1 ? 1 : (k <= 2 ? 2 : (k <= 4 ? 4 : 8)); }

// Median of three unsigned words (v_med3_u32).
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

// Order codes of the two bf16 values of a word, in place: 0x8000 + m for +m and
// 0x8000 - m for -m (so -0 and +0 share 0x8000), computed with packed 16-bit ops.
__device__ __forceinline__ uint32_t order_codes(uint32_t w) {
    const u16x2 x = __builtin_bit_cast(u16x2, w);
    const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, x) >> (int16_t)15);
    const u16x2 mag = (x ^ s) - s;  // 0 - x for negative values, x otherwise
    return __builtin_bit_cast(uint32_t, mag) ^ (~__builtin_bit_cast(uint32_t, s) & 0x80008000u);
}

// One token's E logits are spread over kLanes = E / kPer lanes, kPer = min(E, 32)
// logits (kPer / 8 16-byte loads) per lane; a wave handles 64 / kLanes tokens per
// step.  Each lane keeps its KP = next_pow2(K) largest keys (KP <= 8 <= kPer), then
// K rounds pick the largest head across the token's lanes.
template <int E, int K>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const uint16_t* __restrict__ logits,
                                                           int64_t num_tokens,
                                                           int32_t* __restrict__ indices,
                                                           uint16_t* __restrict__ weights) {
    constexpr int kPer = E < 32 ? E : 32;
    constexpr int kLanes = E / kPer;
    constexpr int kGroups = kPer / 8;
    constexpr int KP = next_pow2(K);
    constexpr int kTokensPerWave = 64 / kLanes;
    const int lane = threadIdx.x % 64;
    const int sub = lane % kLanes, grp = lane / kLanes;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
    const int64_t waves = (int64_t)gridDim.x * blockDim.x / 64;
    // the wave's token rows, 64 * kGroups 16-byte pieces, staged through its LDS slice
    __shared__ u32x4 stage[4][64 * kGroups];
    u32x4* mine_lds = stage[threadIdx.x / 64];
    const int64_t total16 = num_tokens * (E / 8);  // 16-byte pieces of the whole input
    // uniform over the wave: every lane takes part in the cross-lane maxima
    for (int64_t t0 = wave * kTokensPerWave; t0 < num_tokens; t0 += waves * kTokensPerWave) {
        const int64_t t = t0 + grp;
        const bool ok = t < num_tokens;
        // nontemporal loads, each instruction one contiguous 1 KB of the wave's rows
        const int64_t p0 = t0 * (E / 8);
        u32x4 ld[kGroups];
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const int64_t pi = p0 + q * 64 + lane;
            ld[q] = pi < total16 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(logits) + pi)
                                 : u32x4{0u, 0u, 0u, 0u};
        }
        wave_lds_sync();  // the previous step's reads of the slice are done
#pragma unroll
        for (int q = 0; q < kGroups; ++q) mine_lds[q * 64 + lane] = ld[q];
        wave_lds_sync();
        u32x4 raw[kGroups];
#pragma unroll
        for (int q = 0; q < kGroups; ++q) raw[q] = mine_lds[grp * (E / 8) + (kPer / 8) * sub + q];
        uint32_t top[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) top[i] = 0u;  // below every key
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // low half: 31 - (position in the lane); made global after selection
                const uint32_t code = order_codes(raw[q][e]);
                const uint32_t key_lo = (code << 16) | (uint32_t)(31 - (8 * q + 2 * e));
                const uint32_t key_hi = (code & 0xFFFF0000u) | (uint32_t)(30 - (8 * q + 2 * e));
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const uint32_t x = h2 ? key_hi : key_lo;
                    // insert x into the descending list: entry i becomes the median of
                    // old entries i-1, i and x (the list's top: the larger of two)
#pragma unroll
                    for (int i = KP - 1; i >= 1; --i) top[i] = med3_u32(top[i - 1], top[i], x);
                    top[0] = max(top[0], x);
                }
            }
        }
        // low half 31 - pos becomes 0xFFFF - expert with expert = kPer * sub + pos (no
        // carry); every entry is a real key, since KP <= 8 <= kPer
        const uint32_t to_global = 0xFFFFu - (uint32_t)(kPer * sub) - 31u;
#pragma unroll
        for (int i = 0; i < KP; ++i) top[i] += to_global;
        // round r: the largest head among the token's lanes wins; its lane moves on
        uint32_t win[K];
#pragma unroll
        for (int r = 0; r < K; ++r) {
            const uint32_t best = group_max<kLanes>(top[0]);
            win[r] = best;
            const bool mine = top[0] == best;  // keys are distinct (expert index)
#pragma unroll
            for (int j = 0; j < K - 1 - r; ++j) top[j] = mine ? top[j + 1] : top[j];
            top[K - 1 - r] = mine ? 0u : top[K - 1 - r];
        }
        // softmax over the K winners (all lanes of the token hold them)
        const float z0 = code_value(win[0] >> 16);
        float e[K], sum = 0.0f;
#pragma unroll
        for (int r = 0; r < K; ++r) {
            e[r] = fast_exp2((code_value(win[r] >> 16) - z0) * kLog2e);
            sum += e[r];
        }
        const float inv = 1.0f / sum;
        if (ok && sub == 0) {
#pragma unroll
            for (int r = 0; r < K; ++r) {
                indices[t * K + r] = (int32_t)(0xFFFFu - (win[r] & 0xFFFFu));
                weights[t * K + r] = f32_to_bf16_bits(e[r] * inv);
            }
        }
    }
}

template <int E>
hipError_t launch_experts(const void* logits, int64_t num_tokens, int k, int32_t* indices,
                          void* weights, hipStream_t stream) {
    constexpr int kLanes = E / (E < 32 ? E : 32);
    constexpr int kTokensPerBlock = 4 * (64 / kLanes);
    const int64_t need = (num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
    const dim3 grid((unsigned)(need < 65536 ? need : 65536));
    const uint16_t* lg = static_cast<const uint16_t*>(logits);
    uint16_t* w = static_cast<uint16_t*>(weights);
    switch (k) {
#define SA_CASE(KK) case KK: hipLaunchKernelGGL((topk_softmax_kernel<E, KK>), grid, dim3(256), 0, stream, lg, num_tokens, indices, w); break;
        SA_CASE(1) SA_CASE(2) SA_CASE(3) SA_CASE(4) SA_CASE(5) SA_CASE(6) SA_CASE(7) SA_CASE(8)
#undef SA_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_softmax(const void* logits, int64_t num_tokens, int num_experts, int k,
                               int32_t* indices, void* weights, hipStream_t stream) {
    switch (num_experts) {
        case 8: return launch_experts<8>(logits, num_tokens, k, indices, weights, stream);
        case 16: return launch_experts<16>(logits, num_tokens, k, indices, weights, stream);
        case 32: return launch_experts<32>(logits, num_tokens, k, indices, weights, stream);
        case 64: return launch_experts<64>(logits, num_tokens, k, indices, weights, stream);
        case 128: return launch_experts<128>(logits, num_tokens, k, indices, weights, stream);
        case 256: return launch_experts<256>(logits, num_tokens, k, indices, weights, stream);
        case 512: return launch_experts<512>(logits, num_tokens, k, indices, weights, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sa
