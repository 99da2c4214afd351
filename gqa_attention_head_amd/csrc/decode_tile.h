// One wave's split-KV decode step on gfx950 matrix cores: up to 16 query columns
// (query heads, or query rows x heads) of one KV head against 32-key tiles of K/V.
// Shared by the split-KV decode pass and the short-query path of prefill.
//
// Per 32-key tile and wave:
//   S^T[32 keys x 16 columns] = K[32 x 64] . Q^T[64 x 16]      4 MFMA 16x16x32
//     (A = K rows loaded from global memory directly in operand layout,
//      B = the query columns zero-padded to 16; lane (q4, c16) then holds 4+4
//      scores of column c16)
//   online-softmax update in base 2 (scores multiplied by sm_scale * log2 e)
//   O^T[64 dims x 16 columns] += V^T[64 x 32] . P^T[32 x 16]  4 MFMA 16x16x32
//     (V staged row-major in this wave's LDS slice and read back transposed with
//      ds_read_b64_tr_b16; P^T is the exponentiated S^T tile converted to bf16)
#pragma once

#include "common.h"

namespace sa {

constexpr int kDecodeTileKeys = 32;     // keys per wave iteration
constexpr int kDecodeVStride = 64 + 8;  // LDS row stride of a wave's V slice, bf16 elements
// bf16 elements of one wave's V slice in LDS
constexpr int kDecodeVSlice = kDecodeTileKeys * kDecodeVStride;

struct DecodeTile {
    bf16x8 ka[2][2];   // K operand: [key block][dim half]
    u32x4 vr[4];       // four 16-byte V segments (rows lane/8 + 8r)
};

template <bool kStream>
__device__ __forceinline__ u32x4 load_kv(const uint16_t* p) {
    return kStream ? load_stream(p) : *reinterpret_cast<const u32x4*>(p);
}

// Keys t0 .. t0 + 31 of K and V (row pitch row_stride elements), clamped to key hi - 1.
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
    float m;       // running max, base 2 (uniform over the 4 lane groups of a column)
    float dl;      // this lane's share of the running scale
    f32x4 o[4];    // O^T[dim 16*mt + 4*q4 + i][column c16]
};

// One tile: keys at or past lim (per lane, so per column) are masked out.
__device__ __forceinline__ void process_tile(WaveState& st, const DecodeTile& cur, bf16x8 qb0,
                                             bf16x8 qb1, uint16_t* vw, int t0, int lim,
                                             float scale_log2, int lane) {
    const int q4 = lane / 16, c16 = lane % 16;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = mfma16x16x32(cur.ka[0][0], qb0, s0);
    s0 = mfma16x16x32(cur.ka[0][1], qb1, s0);
    s1 = mfma16x16x32(cur.ka[1][0], qb0, s1);
    s1 = mfma16x16x32(cur.ka[1][1], qb1, s1);

#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(vw + (lane / 8 + 8 * r) * kDecodeVStride + 8 * (lane % 8)) = cur.vr[r];

    // s0[i]: key t0 + 4*q4 + i; s1[i]: key t0 + 16 + 4*q4 + i; column c16.
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (t0 + 4 * q4 + i < lim) ? s0[i] * scale_log2 : kNegInf;
        x[4 + i] = (t0 + 16 + 4 * q4 + i < lim) ? s1[i] * scale_log2 : kNegInf;
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
        const uint16_t* p0 = vw + (4 * q4 + c16 / 4) * kDecodeVStride + 16 * mt + 4 * (c16 % 4);
        const bf16x8 va = concat(lds_read_tr16(p0), lds_read_tr16(p0 + 16 * kDecodeVStride));
        st.o[mt] = mfma16x16x32(va, pb, st.o[mt]);
    }
}

}  // namespace sa
