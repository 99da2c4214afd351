// Pre-attention epilogue (gfx950): QKV bias add and rotary position embedding.
//
// "GPT-OSS on day 0" (Perplexity), architecture list: the QKV projections carry
// biases and positions are encoded with YaRN rotary embeddings.  The YaRN
// frequencies and attention scale come folded into a per-position table (row p:
// cos(p w_i) for i < 32, then sin(p w_i)); this kernel adds the bias to every
// head of a token, rotates the query and key heads by their token's table row
// (rotate-halves pairing: element i with element i + 32) and writes q, k and v
// in the [token, head, 64] layouts the attention entry points read.
//
// Layout: the projection output is streamed as 16-byte pieces, eight per head,
// piece p of a head holding elements 8p .. 8p+7 in lane p of an aligned group of
// eight lanes, so every load and store instruction of a wave covers whole
// 128-byte head rows (1 KB contiguous).  The rotation partner of piece p < 4 is
// piece p + 4, one lane-xor-4 swizzle away.  Each thread handles two pieces 256
// apart, and both loads are issued before either is used.  The projection output
// and q/k/v are touched once (nontemporal); bias and table rows stay cached.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kItems = 2;  // pieces per thread

__device__ __forceinline__ void unpack8(u32x4 w, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ u32x4 pack8(const float* y) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)f32_to_bf16_bits(y[2 * e]) | ((uint32_t)f32_to_bf16_bits(y[2 * e + 1]) << 16);
    return w;
}

__global__ __launch_bounds__(256) void qkv_rope_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ bias,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin,
    int64_t num_tokens, int hq, int hkv, int rows, uint16_t* __restrict__ q,
    uint16_t* __restrict__ k, uint16_t* __restrict__ v) {
    const int heads = hq + 2 * hkv;
    const int64_t total = num_tokens * heads * 8;  // 16-byte pieces
    const int64_t base = (int64_t)blockIdx.x * 256 * kItems + threadIdx.x;
    u32x4 raw[kItems];
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
        const int64_t gid = base + u * 256;
        raw[u] = u32x4{0u, 0u, 0u, 0u};
        if (gid < total) raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qkv) + gid);
    }
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
        const int64_t gid = base + u * 256;
        const int piece = (int)(gid % 8);
        const int64_t rest = gid / 8;
        const int hh = (int)(rest % heads);
        const int64_t t = rest / heads;
        const bool live = gid < total;  // uniform over each group of eight lanes
        float x[8], b[8];
        unpack8(raw[u], x);
        unpack8(*reinterpret_cast<const u32x4*>(bias + hh * kD + 8 * piece), b);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += b[e];
        // every lane takes part in the exchange: partner = lane ^ 4 (same head)
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pr[e] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[e]), 0x101F));
        if (live && hh < hq + hkv) {  // query or key head: rotate
            const int p = min(max(positions[t], 0), rows - 1);
            const int i = piece % 4;
            const float* row = cos_sin + (int64_t)p * kD;
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(row + 8 * i);
            const f32x4 c1 = *reinterpret_cast<const f32x4*>(row + 8 * i + 4);
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(row + 32 + 8 * i);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(row + 32 + 8 * i + 4);
            // low half: x c - partner s; high half: x c + partner s
            const float sign = piece < 4 ? -1.0f : 1.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float c = (e < 4) ? c0[e] : c1[e - 4];
                const float s = (e < 4) ? s0[e] : s1[e - 4];
                x[e] = __builtin_fmaf(x[e], c, sign * (pr[e] * s));
            }
        }
        if (!live) continue;
        uint16_t* dst;
        if (hh < hq)
            dst = q + (t * hq + hh) * kD;
        else if (hh < hq + hkv)
            dst = k + (t * hkv + (hh - hq)) * kD;
        else
            dst = v + (t * hkv + (hh - hq - hkv)) * kD;
        __builtin_nontemporal_store(pack8(x), reinterpret_cast<u32x4*>(dst + 8 * piece));
    }
}

}  // namespace

hipError_t launch_qkv_rope(const void* qkv, const void* bias, const int32_t* positions,
                           const float* cos_sin, int64_t num_tokens, int hq, int hkv, int rows,
                           void* q, void* k, void* v, hipStream_t stream) {
    const int64_t pieces = num_tokens * (hq + 2 * hkv) * 8;
    const int64_t blocks = (pieces + 256 * kItems - 1) / (256 * kItems);
    hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(bias),
                       positions, cos_sin, num_tokens, hq, hkv, rows, static_cast<uint16_t*>(q),
                       static_cast<uint16_t*>(k), static_cast<uint16_t*>(v));
    return hipGetLastError();
}

}  // namespace sa
