// Vector-ALU attention-with-sink kernel: one lane per (query row, query head),
// float32 arithmetic throughout.  It serves the float32 path (where the
// tolerance asks for true fp32 products, not bf16 matrix cores) and any
// grouped-query layout the matrix-core kernels do not cover.
//
// Method ("GPT-OSS on day 0", Kernels for GPT-OSS / Sink attention): online
// softmax with a running maximum m and running scale d; m starts at the head's
// sink (scaled into base-2 units) in the first block of keys only, d at 1.
// Scores are kept in base 2: x = <q, k> * sm_scale * log2(e), so e^(s - m)
// becomes 2^(x - m2) and the sink enters as sink * log2(e).
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kTileKeys = 32;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_bits_to_f32(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16_bits(x); }

// What a launch computes: the whole attention of blocks of query rows (kRows),
// the chunk states of single-query sequences (kDecodeSplit), or the chunk states
// of blocks of query rows (kRowsSplit: one key chunk per launch index).
enum Mode { kRows, kDecodeSplit, kRowsSplit };

// grid.x: block of query rows (kRows, kRowsSplit) or key chunk (kDecodeSplit);
// grid.y: KV head; grid.z: sequence (kRowsSplit: sequence * ss.n_chunks + chunk).
// Split modes write chunk c's state of row r to slot r * ss.stride + ss.slot0 + c;
// the sink enters chunk 0 when ss.sink is set.
template <typename T, Mode kMode>
__global__ __launch_bounds__(64) void rows_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ sinks, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int hq, int hkv, float scale_log2, int causal,
    StateSlots ss, T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_m,
    float* __restrict__ part_d, float* __restrict__ part_acc) {
    __shared__ float ks[kTileKeys][kD];
    __shared__ float vs[kTileKeys][kD];

    const int group = hq / hkv;
    const int rows_per_wave = 64 / group;
    const int lane = threadIdx.x;
    constexpr bool kSplit = kMode != kRows;
    const int g = blockIdx.y;
    const int b = (kMode == kRowsSplit) ? blockIdx.z / ss.n_chunks : blockIdx.z;
    const int r_local = lane / group, hh = lane % group;
    const int h = g * group + hh;

    const int k0 = cu_k[b];
    const int lk = cu_k[b + 1] - k0;
    int lq, row, key_lo, key_hi;
    bool first_block;
    if (kMode == kDecodeSplit) {
        lq = 1;
        row = r_local;  // one query per sequence: only lanes with r_local == 0 are active
        const int c = blockIdx.x;
        const int nch = max(1, ceil_div(lk, ss.chunk));
        if (c >= nch) return;
        key_lo = c * ss.chunk;
        key_hi = min(key_lo + ss.chunk, lk);
        first_block = (c == 0 && ss.sink != 0);
    } else {
        const int q0 = cu_q[b];
        lq = cu_q[b + 1] - q0;
        const int r0 = blockIdx.x * rows_per_wave;
        if (r0 >= lq) return;
        row = r0 + r_local;
        const int last = min(r0 + rows_per_wave, lq) - 1;
        key_lo = 0;
        key_hi = causal ? max(0, min(lk, lk - lq + last + 1)) : lk;
        first_block = true;
        if (kMode == kRowsSplit) {  // this launch index's chunk of the keys
            const int c = blockIdx.z % ss.n_chunks;
            key_lo = c * ss.chunk;
            key_hi = min(key_hi, key_lo + ss.chunk);
            first_block = (c == 0 && ss.sink != 0);
        }
    }
    const bool active = (r_local < rows_per_wave) && (row < lq);
    // last key (exclusive) this row may see
    const int row_limit = (kMode != kDecodeSplit && causal) ? min(key_hi, lk - lq + row + 1) : key_hi;

    float qr[kD];
    {
        const int64_t qrow = (kMode == kDecodeSplit) ? (int64_t)b : (int64_t)(cu_q[b] + min(row, lq - 1));
        const T* qp = q + (qrow * hq + (active ? h : g * group)) * kD;
#pragma unroll
        for (int d = 0; d < kD; ++d) qr[d] = to_f32<T>(qp[d]) * scale_log2;
    }
    float m = (first_block && active) ? sinks[h] * kLog2e : kNegInf;
    // the scale starts at 1 with the sink; an empty chunk state has scale 0
    float dsum = (first_block || kMode == kDecodeSplit) ? 1.0f : 0.0f;
    float acc[kD];
#pragma unroll
    for (int d = 0; d < kD; ++d) acc[d] = 0.0f;

    for (int t0 = key_lo; t0 < key_hi; t0 += kTileKeys) {
        __syncthreads();
        for (int idx = lane; idx < kTileKeys * kD; idx += 64) {
            const int j = idx / kD, d = idx % kD;
            const int key = min(t0 + j, key_hi - 1);
            const int64_t off = ((int64_t)(k0 + key) * hkv + g) * kD + d;
            ks[j][d] = to_f32<T>(k[off]);
            vs[j][d] = to_f32<T>(v[off]);
        }
        __syncthreads();
        float s[kTileKeys];
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < kTileKeys; ++j) {
            float x = 0.0f;
#pragma unroll
            for (int d = 0; d < kD; ++d) x = fmaf(qr[d], ks[j][d], x);
            const bool ok = (t0 + j < row_limit);
            s[j] = ok ? x : kNegInf;
            tmax = fmaxf(tmax, s[j]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new != kNegInf) {
            const float alpha = fast_exp2(m - m_new);
            float psum = 0.0f;
#pragma unroll
            for (int d = 0; d < kD; ++d) acc[d] *= alpha;
#pragma unroll
            for (int j = 0; j < kTileKeys; ++j) {
                const float p = fast_exp2(s[j] - m_new);
                psum += p;
#pragma unroll
                for (int d = 0; d < kD; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
            }
            dsum = dsum * alpha + psum;
            m = m_new;
        }
    }
    if (!active) return;

    if (kSplit) {
        const int c = (kMode == kDecodeSplit) ? blockIdx.x : blockIdx.z % ss.n_chunks;
        const int64_t srow = (kMode == kDecodeSplit) ? (int64_t)b : (int64_t)cu_q[b] + row;
        const int64_t slot = (srow * hq + h) * ss.stride + ss.slot0 + c;
        part_m[slot] = (m == kNegInf) ? kNegInf : m * kLn2;
        part_d[slot] = dsum;
        float* pa = part_acc + slot * kD;
#pragma unroll
        for (int d = 0; d < kD; ++d) pa[d] = acc[d];
    } else {
        const int64_t orow = (int64_t)cu_q[b] + row;
        T* op = out + (orow * hq + h) * kD;
        if (m == kNegInf) {
#pragma unroll
            for (int d = 0; d < kD; ++d) op[d] = from_f32<T>(0.0f);
            if (lse) lse[orow * hq + h] = kNegInf;
        } else {
            const float inv = 1.0f / dsum;
#pragma unroll
            for (int d = 0; d < kD; ++d) op[d] = from_f32<T>(acc[d] * inv);
            if (lse) lse[orow * hq + h] = (m + fast_log2(dsum)) * kLn2;
        }
    }
}

}  // namespace

hipError_t launch_generic_prefill(bool bf16, const void* q, const void* k, const void* v,
                                  const float* sinks, const int32_t* cu_q, const int32_t* cu_k,
                                  int batch, int hq, int hkv, int max_lq, float sm_scale,
                                  int causal, void* out, float* lse, hipStream_t stream) {
    const int group = hq / hkv;
    const int rows_per_wave = 64 / group;
    dim3 grid(ceil_div(max_lq, rows_per_wave), hkv, batch);
    const float sl = sm_scale * kLog2e;
    if (bf16)
        hipLaunchKernelGGL((rows_kernel<uint16_t, kRows>), grid, dim3(64), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks, cu_q,
                           cu_k, hq, hkv, sl, causal, StateSlots{0, 1, 1, 0, 1}, (uint16_t*)out,
                           lse, nullptr, nullptr, nullptr);
    else
        hipLaunchKernelGGL((rows_kernel<float, kRows>), grid, dim3(64), 0, stream, (const float*)q,
                           (const float*)k, (const float*)v, sinks, cu_q, cu_k, hq, hkv, sl, causal,
                           StateSlots{0, 1, 1, 0, 1}, (float*)out, lse, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_generic_decode_split(bool bf16, const void* q, const void* k, const void* v,
                                       const float* sinks, const int32_t* cu_k, int batch, int hq,
                                       int hkv, int chunk, int max_chunks, float sm_scale,
                                       float* part_m, float* part_d, float* part_acc,
                                       hipStream_t stream) {
    dim3 grid(max_chunks, hkv, batch);
    const float sl = sm_scale * kLog2e;
    const StateSlots ss{chunk, max_chunks, max_chunks, 0, 1};
    if (bf16)
        hipLaunchKernelGGL((rows_kernel<uint16_t, kDecodeSplit>), grid, dim3(64), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks,
                           nullptr, cu_k, hq, hkv, sl, 0, ss, nullptr, nullptr, part_m, part_d,
                           part_acc);
    else
        hipLaunchKernelGGL((rows_kernel<float, kDecodeSplit>), grid, dim3(64), 0, stream, (const float*)q,
                           (const float*)k, (const float*)v, sinks, nullptr, cu_k, hq, hkv, sl, 0,
                           ss, nullptr, nullptr, part_m, part_d, part_acc);
    return hipGetLastError();
}

hipError_t launch_generic_prefill_split(bool bf16, const void* q, const void* k, const void* v,
                                        const float* sinks, const int32_t* cu_q,
                                        const int32_t* cu_k, int batch, int hq, int hkv,
                                        int max_lq, const StateSlots& ss, float sm_scale,
                                        int causal, float* part_m, float* part_d,
                                        float* part_acc, hipStream_t stream) {
    const int group = hq / hkv;
    const int rows_per_wave = 64 / group;
    dim3 grid(ceil_div(max_lq, rows_per_wave), hkv, batch * ss.n_chunks);
    const float sl = sm_scale * kLog2e;
    if (bf16)
        hipLaunchKernelGGL((rows_kernel<uint16_t, kRowsSplit>), grid, dim3(64), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks, cu_q,
                           cu_k, hq, hkv, sl, causal, ss, nullptr, nullptr, part_m, part_d,
                           part_acc);
    else
        hipLaunchKernelGGL((rows_kernel<float, kRowsSplit>), grid, dim3(64), 0, stream,
                           (const float*)q, (const float*)k, (const float*)v, sinks, cu_q, cu_k, hq,
                           hkv, sl, causal, ss, nullptr, nullptr, part_m, part_d, part_acc);
    return hipGetLastError();
}

}  // namespace sa
