// Split-KV decode, first pass, bf16 inputs, head_dim 64, matrix cores (gfx950).
//
// "GPT-OSS on day 0" (Perplexity), Kernels for GPT-OSS / Sink attention:
// attention is parallelised across independent heads and along the KV
// sequence; the online softmax keeps a running maximum m and a running scale
// d; m starts at the head's sink in the first block of keys only.  This kernel
// writes, for every (sequence b, chunk c, query head h), the state (m, d, acc)
// after chunk c's keys.
//
// Work decomposition (HBM-bound: every K/V byte is read exactly once).
// One workgroup per (b, c, block of up to 8 KV heads); wave w of the
// workgroup owns KV head g = 8*block + w and the G query heads that share it.
// K/V are token-major ([token][kv head][64]), so the 8 waves together stream
// whole contiguous 1 KB token rows: workgroups never read a fraction of a
// DRAM row that another workgroup reads later.  Each wave keeps kDepth tiles
// of loads in flight in registers, read with nontemporal loads.  Above 16 query
// heads per KV head, the heads are cut into slices of G, one wave each; the waves
// of one KV head then read the same K/V rows, with cached loads so that the later
// ones hit in the cache.
//
//
// Per 32-key tile and wave:
//   S^T[32 keys x 16 heads] = K[32 x 64] . Q^T[64 x 16]      4 MFMA 16x16x32
//     (A = K rows loaded from global memory directly in operand layout,
//      B = the G <= 16 query heads zero-padded to 16 columns; lane (q4, c16)
//      then holds 4+4 scores of head c16)
//   online-softmax update in base 2 (scores pre-multiplied by sm_scale*log2 e)
//   O^T[64 dims x 16 heads] += V^T[64 x 32] . P^T[32 x 16]  4 MFMA 16x16x32
//     (V staged row-major in this wave's LDS slice and read back transposed
//      with ds_read_b64_tr_b16; P^T is the exponentiated S^T tile converted to
//      bf16 in place)
#include "common.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kTile = 32;            // keys per wave iteration
constexpr int kVStride = kD + 8;     // LDS row stride in bf16 elements (144 bytes)

struct DecodeTile {
    bf16x8 ka[2][2];   // K operand: [key block][dim half]
    u32x4 vr[4];       // four 16-byte V segments (rows lane/8 + 8r)
};

template <bool kStream>
__device__ __forceinline__ u32x4 load_kv(const uint16_t* p) {
    return kStream ? load_stream(p) : *reinterpret_cast<const u32x4*>(p);
}

template <bool kStream>
__device__ __forceinline__ void load_tile(DecodeTile& t, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int row_stride,
                                          int t0, int hi, int lane) {
    const int q4 = lane / 16, c16 = lane % 16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int key = min(t0 + 16 * kb + c16, hi - 1);
        const uint16_t* kp = kbase + (int64_t)key * row_stride + 8 * q4;
        t.ka[kb][0] = __builtin_bit_cast(bf16x8, load_kv<kStream>(kp));
        t.ka[kb][1] = __builtin_bit_cast(bf16x8, load_kv<kStream>(kp + 32));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = min(t0 + lane / 8 + 8 * r, hi - 1);
        t.vr[r] = load_kv<kStream>(vbase + (int64_t)key * row_stride + 8 * (lane % 8));
    }
    // Keep the loads where they are issued: the scheduler would otherwise move
    // them next to their first use and the prefetch would be lost.
    __builtin_amdgcn_sched_barrier(0);
}

struct WaveState {
    float m;       // running max, base 2 (uniform over the 4 lane groups of a head column)
    float dl;      // this lane's share of the running scale
    f32x4 o[4];    // O^T[dim 16*mt + 4*q4 + i][head c16]
};

__device__ __forceinline__ void process_tile(WaveState& st, const DecodeTile& cur, bf16x8 qb0,
                                             bf16x8 qb1, uint16_t* vw, int t0, int hi,
                                             float scale_log2, int lane) {
    const int q4 = lane / 16, c16 = lane % 16;
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
    const float m_new = fmaxf(st.m, tmax);
    const bool live = m_new != kNegInf;
    const float alpha = live ? fast_exp2(st.m - m_new) : 1.0f;
    const float msub = live ? m_new : 0.0f;
    float psum = 0.0f;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(x[i] - msub);
        psum += p;
        pb[i] = static_cast<__bf16>(p);
    }
    st.dl = st.dl * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.o[mt] *= alpha;

    wave_lds_sync();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const uint16_t* p0 = vw + (4 * q4 + c16 / 4) * kVStride + 16 * mt + 4 * (c16 % 4);
        const bf16x8 va = concat(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * kVStride));
        st.o[mt] = mfma16x16x32(va, pb, st.o[mt]);
    }
}

template <int G, int kDepth, int kHeadsPerBlock, bool kHeadSlices = false>
__global__ __launch_bounds__(64 * kHeadsPerBlock) void decode_split_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_k, int hq, int hkv, int chunk, int max_chunks,
    int head_blocks, float scale_log2, float* __restrict__ part_m,
    float* __restrict__ part_d, float* __restrict__ part_acc) {
    __shared__ uint16_t vlds[kHeadsPerBlock][kTile * kVStride];

    // blockIdx -> (b, chunk c, head block hb), head block fastest
    const int hb = blockIdx.x % head_blocks;
    const int t = blockIdx.x / head_blocks;
    const int c = t % max_chunks;
    const int b = t / max_chunks;
    const int k0 = cu_k[b];
    const int len = cu_k[b + 1] - k0;
    // (chunks beyond max_chunks would break the ABI's bound on the sequence
    // length; they are left out rather than written out of range)
    const int nch = min(max_chunks, max(1, ceil_div(len, chunk)));
    if (c >= nch) return;  // uniform over the workgroup
    const int lo = c * chunk;
    const int hi = min(lo + chunk, len);

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    // kHeadSlices: more than 16 query heads share a KV head; wave unit u covers
    // slice u % slices (G heads) of KV head u / slices.
    const int group = kHeadSlices ? hq / hkv : G;
    const int slices = group / G;
    const int u = hb * kHeadsPerBlock + wave;
    const int g = kHeadSlices ? u / slices : u;
    const int hs = kHeadSlices ? u % slices : 0;
    const bool g_ok = g < hkv;
    const int q4 = lane / 16, c16 = lane % 16;
    const bool head_ok = g_ok && c16 < G;
    const int h = g * group + hs * G + c16;
    const int row_stride = hkv * kD;
    const int gsafe = g_ok ? g : 0;
    const uint16_t* kbase = k + ((int64_t)k0 * hkv + gsafe) * kD;
    const uint16_t* vbase = v + ((int64_t)k0 * hkv + gsafe) * kD;

    // m starts at the sink in chunk 0 only; the scale starts at 1, held by one
    // lane share (q4 == 0).
    WaveState st;
    st.m = (c == 0 && head_ok) ? sinks[h] * kLog2e : kNegInf;
    st.dl = (q4 == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint16_t* vw = vlds[wave];
    const int ntiles = (g_ok && lo < hi) ? ceil_div(hi - lo, kTile) : 0;
    // B operand of S^T = K Q^T: lane holds Q[head c16][dims 8*q4 .. +7] (and +32).
    bf16x8 qb0 = {}, qb1 = {};
    if (head_ok) {
        const uint16_t* qp = q + ((int64_t)b * hq + h) * kD + 8 * q4;
        qb0 = load_bf16x8(qp);
        qb1 = load_bf16x8(qp + 32);
    }

    // kDepth tiles of loads stay in flight per wave.  Loads are issued
    // unconditionally (addresses clamped to the chunk's last key, which exists
    // when ntiles > 0), so every tile has exactly the same number of loads
    // issued after it and the wait before a tile covers that tile's loads only;
    // the loop body is branch-free (a tile past the end has every key masked and
    // leaves the state unchanged).
    if (ntiles > 0) {
        DecodeTile buf[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            load_tile<!kHeadSlices>(buf[d], kbase, vbase, row_stride, lo + d * kTile, hi, lane);
        int it = 0;
        do {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int ts = lo + (it + d) * kTile;
                process_tile(st, buf[d], qb0, qb1, vw, ts, hi, scale_log2, lane);
                load_tile<!kHeadSlices>(buf[d], kbase, vbase, row_stride, ts + kDepth * kTile, hi, lane);
            }
            it += kDepth;
        } while (it < ntiles);
    }

    // Reduce the scale over the four lane groups of each head column.
    st.dl += xor16(st.dl);
    st.dl = sum_xor32(st.dl);

    const float m_nat = (st.m == kNegInf) ? kNegInf : st.m * kLn2;
    const int64_t slot = ((int64_t)b * hq + h) * max_chunks + c;
    if (head_ok) {
        float* pa = part_acc + slot * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(pa + 16 * mt + 4 * q4) = st.o[mt];
        if (q4 == 0) {
            part_m[slot] = m_nat;
            part_d[slot] = st.dl;
        }
    }
}

template <int G, bool kHeadSlices>
hipError_t launch_g(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_k, int batch, int hq, int hkv, int chunk, int max_chunks,
                    float sm_scale, float* part_m, float* part_d, float* part_acc,
                    hipStream_t stream) {
    constexpr int kDepth = 2, kHeadsPerBlock = 8;
    const int units = hkv * ((hq / hkv) / G);  // (KV head, slice of G query heads)
    const int head_blocks = ceil_div(units, kHeadsPerBlock);
    const int64_t blocks = (int64_t)batch * max_chunks * head_blocks;
    hipLaunchKernelGGL((decode_split_mfma<G, kDepth, kHeadsPerBlock, kHeadSlices>),
                       dim3((unsigned)blocks), dim3(64 * kHeadsPerBlock), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks, cu_k, hq,
                       hkv, chunk, max_chunks, head_blocks, sm_scale * kLog2e, part_m, part_d,
                       part_acc);
    return hipGetLastError();
}

}  // namespace

bool mfma_decode_supported(int group) { return group >= 1 && group <= 64; }

hipError_t launch_mfma_decode_split(const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_k, int batch, int hq,
                                    int hkv, int chunk, int max_chunks, float sm_scale,
                                    float* part_m, float* part_d, float* part_acc,
                                    hipStream_t stream) {
    const int group = hq / hkv;
#define SA_ARGS q, k, v, sinks, cu_k, batch, hq, hkv, chunk, max_chunks, sm_scale, part_m, part_d, part_acc, stream
    switch (group) {
#define SA_CASE(GG) case GG: return launch_g<GG, false>(SA_ARGS);
        SA_CASE(1) SA_CASE(2) SA_CASE(3) SA_CASE(4) SA_CASE(5) SA_CASE(6) SA_CASE(7) SA_CASE(8)
        SA_CASE(9) SA_CASE(10) SA_CASE(11) SA_CASE(12) SA_CASE(13) SA_CASE(14) SA_CASE(15) SA_CASE(16)
#undef SA_CASE
        default: break;
    }
    // more than 16 heads per KV head: slices of the largest divisor of the group
    // that is at most 16 and a power of two (one wave per slice)
    if (group > 16 && group <= 64) {
        if (group % 16 == 0) return launch_g<16, true>(SA_ARGS);
        if (group % 8 == 0) return launch_g<8, true>(SA_ARGS);
        if (group % 4 == 0) return launch_g<4, true>(SA_ARGS);
        if (group % 2 == 0) return launch_g<2, true>(SA_ARGS);
        return launch_g<1, true>(SA_ARGS);
    }
#undef SA_ARGS
    return hipErrorInvalidValue;
}

}  // namespace sa
