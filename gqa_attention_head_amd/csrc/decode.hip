// Split-KV decode, first pass, bf16 inputs, head_dim 64, matrix cores (gfx950).
//
// "GPT-OSS on day 0" (Perplexity), Kernels for GPT-OSS / Sink attention:
// attention is parallelised across independent heads and along the KV
// sequence; the online softmax keeps a running maximum m and a running scale
// d; m starts at the head's sink in the first block of keys only.  This kernel
// computes, for one (sequence b, KV head g, chunk c), the state (m, d, acc) of
// all G query heads that share KV head g after the chunk's keys.
//
// Work decomposition.  One workgroup of 4 waves per (b, g, c).  The chunk's
// keys are cut into 32-key tiles dealt round-robin to the waves, so the four
// waves stream neighbouring K/V rows at the same time.  Each wave keeps its
// own online-softmax state; the four states are combined through LDS at the
// end (the same log-sum-exp rule the merge pass uses).
//
// Per 32-key tile and wave:
//   S^T[32 keys x 16 heads] = K[32 x 64] . Q^T[64 x 16]      2+2 MFMA 16x16x32
//     (A = K rows straight from global memory in operand layout, B = the G <= 16
//      query heads, zero-padded to 16 columns; lane (q4, c16) ends up holding
//      4+4 scores of head c16)
//   online-softmax update in base 2 (scores pre-multiplied by sm_scale*log2 e)
//   O^T[64 dims x 16 heads] += V^T[64 x 32] . P^T[32 x 16]  4 MFMA 16x16x32
//     (V staged row-major in this wave's LDS slice and read back transposed
//      with ds_read_b64_tr_b16; P^T is the exponentiated S^T tile converted to
//      bf16 in place, no data movement)
// K is half of the bytes and V the other half; both are read exactly once.
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kWaves = 4;
constexpr int kTile = 32;            // keys per wave iteration
constexpr int kVStride = kD + 8;     // LDS row stride in bf16 elements (144 bytes)

struct DecodeTile {
    bf16x8 ka[2][2];   // K operand: [key block][dim half]
    u32x4 vr[4];       // 4 rows' worth of 16-byte V segments
};

__device__ __forceinline__ void load_tile(DecodeTile& t, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int row_stride,
                                          int t0, int hi, int lane) {
    const int q4 = lane / 16, c16 = lane % 16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = min(t0 + 16 * kb + c16, hi - 1);
        const uint16_t* kp = kbase + (int64_t)key * row_stride + 8 * q4;
        t.ka[kb][0] = load_bf16x8(kp);
        t.ka[kb][1] = load_bf16x8(kp + 32);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = min(t0 + lane / 8 + 8 * r, hi - 1);
        t.vr[r] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * row_stride + 8 * (lane % 8));
    }
}

template <int G>
__global__ __launch_bounds__(256) void decode_split_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_k, int hq, int hkv, int chunk, int max_chunks,
    float scale_log2, float* __restrict__ part_m, float* __restrict__ part_d,
    float* __restrict__ part_acc) {
    __shared__ uint16_t vlds[kWaves][kTile * kVStride];
    __shared__ float wm[kWaves][G];
    __shared__ float wd[kWaves][G];
    __shared__ float wacc[kWaves][G][kD];

    // KV head fastest so the workgroups of one (b, c) read whole 1 KB token rows together.
    const int g = blockIdx.x % hkv;
    const int t = blockIdx.x / hkv;
    const int c = t % max_chunks;
    const int b = t / max_chunks;
    const int k0 = cu_k[b];
    const int len = cu_k[b + 1] - k0;
    const int nch = max(1, ceil_div(len, chunk));
    if (c >= nch) return;  // uniform over the workgroup
    const int lo = c * chunk;
    const int hi = min(lo + chunk, len);

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int q4 = lane / 16, c16 = lane % 16;
    const bool head_ok = c16 < G;
    const int h = g * G + c16;
    const int row_stride = hkv * kD;
    const uint16_t* kbase = k + ((int64_t)k0 * hkv + g) * kD;
    const uint16_t* vbase = v + ((int64_t)k0 * hkv + g) * kD;

    // B operand of S^T = K Q^T: lane holds Q[head c16][dims 8*q4 .. +7] (and +32).
    bf16x8 qb0 = {}, qb1 = {};
    if (head_ok) {
        const uint16_t* qp = q + ((int64_t)b * hq + h) * kD + 8 * q4;
        qb0 = load_bf16x8(qp);
        qb1 = load_bf16x8(qp + 32);
    }

    // Running state in base-2 units.  m starts at the sink in chunk 0 only; the
    // scale d (whose initial 1 is the sink's own term) is spread over lanes and
    // waves as partial sums, so exactly one lane per head carries that 1.
    float m = (c == 0 && head_ok) ? sinks[h] * kLog2e : kNegInf;
    float dl = (wave == 0 && q4 == 0) ? 1.0f : 0.0f;
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint16_t* vw = vlds[wave];
    const int stride = kTile * kWaves;
    int t0 = lo + kTile * wave;
    DecodeTile cur;
    if (t0 < hi) load_tile(cur, kbase, vbase, row_stride, t0, hi, lane);
    for (; t0 < hi; t0 += stride) {
        DecodeTile nxt;
        const bool more = t0 + stride < hi;
        if (more) load_tile(nxt, kbase, vbase, row_stride, t0 + stride, hi, lane);

        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        s0 = mfma16x16x32(cur.ka[0][0], qb0, s0);
        s0 = mfma16x16x32(cur.ka[0][1], qb1, s0);
        s1 = mfma16x16x32(cur.ka[1][0], qb0, s1);
        s1 = mfma16x16x32(cur.ka[1][1], qb1, s1);

#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4*>(vw + (lane / 8 + 8 * r) * kVStride + 8 * (lane % 8)) = cur.vr[r];

        // s0[i]: key t0 + 4*q4 + i; s1[i]: key t0 + 16 + 4*q4 + i; column = head c16.
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (t0 + 4 * q4 + i < hi) ? s0[i] * scale_log2 : kNegInf;
            x[4 + i] = (t0 + 16 + 4 * q4 + i < hi) ? s1[i] * scale_log2 : kNegInf;
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        tmax = fmaxf(tmax, xor16(tmax));
        tmax = max_xor32(tmax);
        const float m_new = fmaxf(m, tmax);
        const bool live = m_new != kNegInf;
        const float alpha = live ? fast_exp2(m - m_new) : 1.0f;
        const float msub = live ? m_new : 0.0f;
        float psum = 0.0f;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = fast_exp2(x[i] - msub);
            psum += p;
            pb[i] = static_cast<__bf16>(p);
        }
        dl = dl * alpha + psum;
        m = m_new;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;

        wave_lds_sync();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const uint16_t* p0 = vw + (4 * q4 + c16 / 4) * kVStride + 16 * mt + 4 * (c16 % 4);
            const bf16x8 va = concat(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * kVStride));
            o[mt] = mfma16x16x32(va, pb, o[mt]);
        }
        if (more) cur = nxt;
    }

    // Reduce the scale over the four lane groups of each head column.
    dl += xor16(dl);
    dl = sum_xor32(dl);
    if (head_ok) {
        if (q4 == 0) {
            wm[wave][c16] = m;
            wd[wave][c16] = dl;
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) wacc[wave][c16][16 * mt + 4 * q4 + i] = o[mt][i];
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * kD; idx += 64 * kWaves) {
        const int hh = idx / kD, dim = idx % kD;
        float big = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) big = fmaxf(big, wm[w][hh]);
        const int64_t slot = ((int64_t)b * hq + g * G + hh) * max_chunks + c;
        float dsum = 1.0f, acc = 0.0f;
        if (big != kNegInf) {
            dsum = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float wt = fast_exp2(wm[w][hh] - big);
                dsum += wt * wd[w][hh];
                acc += wt * wacc[w][hh][dim];
            }
        }
        part_acc[slot * kD + dim] = acc;
        if (dim == 0) {
            part_m[slot] = (big == kNegInf) ? kNegInf : big * kLn2;
            part_d[slot] = dsum;
        }
    }
}

template <int G>
hipError_t launch_g(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_k, int batch, int hq, int hkv, int chunk, int max_chunks,
                    float sm_scale, float* part_m, float* part_d, float* part_acc,
                    hipStream_t stream) {
    const int64_t blocks = (int64_t)batch * max_chunks * hkv;
    hipLaunchKernelGGL((decode_split_mfma<G>), dim3((unsigned)blocks), dim3(64 * kWaves), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks,
                       cu_k, hq, hkv, chunk, max_chunks, sm_scale * kLog2e, part_m, part_d,
                       part_acc);
    return hipGetLastError();
}

}  // namespace

bool mfma_decode_supported(int group) {
    return group == 1 || group == 2 || group == 4 || group == 8 || group == 16;
}

hipError_t launch_mfma_decode_split(const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_k, int batch, int hq,
                                    int hkv, int chunk, int max_chunks, float sm_scale,
                                    float* part_m, float* part_d, float* part_acc,
                                    hipStream_t stream) {
    switch (hq / hkv) {
        case 1: return launch_g<1>(q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream);
        case 2: return launch_g<2>(q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream);
        case 4: return launch_g<4>(q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream);
        case 8: return launch_g<8>(q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream);
        case 16: return launch_g<16>(q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sa
