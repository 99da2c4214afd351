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
// Thread (token t, head hh, quarter j): elements 8j .. 8j+7 and 32+8j .. 32+8j+7
// of head hh, so four threads cover a head and a wave sixteen heads.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;

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
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int j = (int)(gid % 4);
    const int64_t rest = gid / 4;
    const int hh = (int)(rest % heads);
    const int64_t t = rest / heads;
    if (t >= num_tokens) return;

    const uint16_t* src = qkv + (t * heads + hh) * kD;
    const uint16_t* bs = bias + (int64_t)hh * kD;
    float lo[8], hi[8], blo[8], bhi[8];
    unpack8(*reinterpret_cast<const u32x4*>(src + 8 * j), lo);
    unpack8(*reinterpret_cast<const u32x4*>(src + 32 + 8 * j), hi);
    unpack8(*reinterpret_cast<const u32x4*>(bs + 8 * j), blo);
    unpack8(*reinterpret_cast<const u32x4*>(bs + 32 + 8 * j), bhi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] += blo[e];
        hi[e] += bhi[e];
    }
    if (hh < hq + hkv) {  // query or key head: rotate
        const int p = min(max(positions[t], 0), rows - 1);
        const float* row = cos_sin + (int64_t)p * kD;
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(row + 8 * j);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(row + 8 * j + 4);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(row + 32 + 8 * j);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(row + 32 + 8 * j + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = (e < 4) ? c0[e] : c1[e - 4];
            const float s = (e < 4) ? s0[e] : s1[e - 4];
            const float a = lo[e], b = hi[e];
            lo[e] = __builtin_fmaf(a, c, -b * s);
            hi[e] = __builtin_fmaf(b, c, a * s);
        }
    }
    uint16_t* dst;
    if (hh < hq)
        dst = q + (t * hq + hh) * kD;
    else if (hh < hq + hkv)
        dst = k + (t * hkv + (hh - hq)) * kD;
    else
        dst = v + (t * hkv + (hh - hq - hkv)) * kD;
    *reinterpret_cast<u32x4*>(dst + 8 * j) = pack8(lo);
    *reinterpret_cast<u32x4*>(dst + 32 + 8 * j) = pack8(hi);
}

}  // namespace

hipError_t launch_qkv_rope(const void* qkv, const void* bias, const int32_t* positions,
                           const float* cos_sin, int64_t num_tokens, int hq, int hkv, int rows,
                           void* q, void* k, void* v, hipStream_t stream) {
    const int64_t threads = num_tokens * (hq + 2 * hkv) * 4;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(bias),
                       positions, cos_sin, num_tokens, hq, hkv, rows, static_cast<uint16_t*>(q),
                       static_cast<uint16_t*>(k), static_cast<uint16_t*>(v));
    return hipGetLastError();
}

}  // namespace sa
