// Vector-ALU attention-with-sink kernel: kP lanes per (query row, query head), each
// holding 64 / kP of the head dimensions, float32 arithmetic throughout.  It serves the float32 path (where the
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

// Element e of a 16-byte piece, widened to fp32.
template <typename T>
__device__ __forceinline__ float piece_elem(const u32x4& w, int e);
template <>
__device__ __forceinline__ float piece_elem<float>(const u32x4& w, int e) {
    return __uint_as_float(w[e]);
}
template <>
__device__ __forceinline__ float piece_elem<uint16_t>(const u32x4& w, int e) {
    const uint32_t word = w[e / 2];
    return bf16_bits_to_f32(static_cast<uint16_t>(e % 2 == 0 ? word & 0xFFFFu : word >> 16));
}

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

// Sum over the kP adjacent lanes of a (row, head) pair (quad permutes: lane ^ 1, lane ^ 2).
template <int kP>
__device__ __forceinline__ float pair_sum(float x) {
    if (kP >= 2)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
    if (kP >= 4)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
    return x;
}

// grid.x: block of query rows (kRows, kRowsSplit) or key chunk (kDecodeSplit);
// grid.y: KV head; grid.z: sequence (kRowsSplit: sequence * ss.n_chunks + chunk).
// Lane = ((row in block) * group + head in group) * kP + part: the kP lanes of a
// (row, head) pair each hold kDL of its dimensions and take partial dot products,
// summed across the pair; each then carries the same softmax state.
// Split modes write chunk c's state of row r to slot r * ss.stride + ss.slot0 + c;
// the sink enters chunk 0 when ss.sink is set.
template <typename T, Mode kMode, int kP>
__global__ __launch_bounds__(64) void rows_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ sinks, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int hq, int hkv, float scale_log2, int causal,
    StateSlots ss, T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_m,
    float* __restrict__ part_d, float* __restrict__ part_acc) {
    __shared__ float ks[kTileKeys][kD];
    __shared__ float vs[kTileKeys][kD];

    constexpr int kDL = kD / kP;  // dimensions per lane
    const int group = hq / hkv;
    const int rows_per_wave = 64 / (group * kP);
    const int lane = threadIdx.x;
    constexpr bool kSplit = kMode != kRows;
    const int g = blockIdx.y;
    const int b = (kMode == kRowsSplit) ? blockIdx.z / ss.n_chunks : blockIdx.z;
    const int pair = lane / kP, part = lane % kP;
    const int d0 = part * kDL;  // this lane's first dimension
    const int r_local = pair / group, hh = pair % group;
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

    float qr[kDL];
    {
        const int64_t qrow = (kMode == kDecodeSplit) ? (int64_t)b : (int64_t)(cu_q[b] + min(row, lq - 1));
        const T* qp = q + (qrow * hq + (active ? h : g * group)) * kD + d0;
#pragma unroll
        for (int d = 0; d < kDL; ++d) qr[d] = to_f32<T>(qp[d]) * scale_log2;
    }
    float m = (first_block && active) ? sinks[h] * kLog2e : kNegInf;
    // the scale starts at 1 with the sink; an empty chunk state has scale 0
    float dsum = (first_block || kMode == kDecodeSplit) ? 1.0f : 0.0f;
    float acc[kDL];
#pragma unroll
    for (int d = 0; d < kDL; ++d) acc[d] = 0.0f;

    // K/V tiles move in 16-byte pieces (4 fp32 or 8 bf16 elements): each lane loads
    // kPieces of each into registers, the next tile's while the current one is used,
    // and widens them to fp32 in LDS.
    constexpr int kPieceElems = 16 / sizeof(T);
    constexpr int kPiecesPerRow = kD / kPieceElems;
    constexpr int kPieces = kTileKeys * kPiecesPerRow / 64;  // per lane, K and V each
    u32x4 kr[kPieces], vr[kPieces];
    auto gload = [&](int t0) {
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int piece = lane + 64 * p;
            const int key = min(t0 + piece / kPiecesPerRow, key_hi - 1);
            const int64_t off =
                ((int64_t)(k0 + key) * hkv + g) * kD + (piece % kPiecesPerRow) * kPieceElems;
            kr[p] = *reinterpret_cast<const u32x4*>(k + off);
            vr[p] = *reinterpret_cast<const u32x4*>(v + off);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int piece = lane + 64 * p;
            const int j = piece / kPiecesPerRow, d = (piece % kPiecesPerRow) * kPieceElems;
#pragma unroll
            for (int e = 0; e < kPieceElems; ++e) {
                ks[j][d + e] = piece_elem<T>(kr[p], e);
                vs[j][d + e] = piece_elem<T>(vr[p], e);
            }
        }
    };
    if (key_lo < key_hi) gload(key_lo);

    for (int t0 = key_lo; t0 < key_hi; t0 += kTileKeys) {
        __syncthreads();  // every lane is done with the previous tile
        lstore();
        __syncthreads();
        if (t0 + kTileKeys < key_hi) gload(t0 + kTileKeys);
        float s[kTileKeys];
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < kTileKeys; ++j) {
            float x = 0.0f;
#pragma unroll
            for (int d = 0; d < kDL; ++d) x = fmaf(qr[d], ks[j][d0 + d], x);
            x = pair_sum<kP>(x);
            const bool ok = (t0 + j < row_limit);
            s[j] = ok ? x : kNegInf;
            tmax = fmaxf(tmax, s[j]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new != kNegInf) {
            const float alpha = fast_exp2(m - m_new);
            float psum = 0.0f;
#pragma unroll
            for (int d = 0; d < kDL; ++d) acc[d] *= alpha;
#pragma unroll
            for (int j = 0; j < kTileKeys; ++j) {
                const float p = fast_exp2(s[j] - m_new);
                psum += p;
#pragma unroll
                for (int d = 0; d < kDL; ++d) acc[d] = fmaf(p, vs[j][d0 + d], acc[d]);
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
        if (part == 0) {
            part_m[slot] = (m == kNegInf) ? kNegInf : m * kLn2;
            part_d[slot] = dsum;
        }
        float* pa = part_acc + slot * kD + d0;
#pragma unroll
        for (int d = 0; d < kDL; ++d) pa[d] = acc[d];
    } else {
        const int64_t orow = (int64_t)cu_q[b] + row;
        T* op = out + (orow * hq + h) * kD + d0;
        if (m == kNegInf) {
#pragma unroll
            for (int d = 0; d < kDL; ++d) op[d] = from_f32<T>(0.0f);
            if (lse && part == 0) lse[orow * hq + h] = kNegInf;
        } else {
            const float inv = 1.0f / dsum;
#pragma unroll
            for (int d = 0; d < kDL; ++d) op[d] = from_f32<T>(acc[d] * inv);
            if (lse && part == 0) lse[orow * hq + h] = (m + fast_log2(dsum)) * kLn2;
        }
    }
}

// Lanes per (row, head) pair: four where a wave holds at least one row of the group
// that way, fewer for the largest groups (rows_per_wave = 64 / (group * kP) >= 1).
int lanes_per_pair(int group) { return group <= 16 ? 4 : group <= 32 ? 2 : 1; }

template <typename T, Mode kMode>
hipError_t launch_rows(dim3 grid, hipStream_t stream, const void* q, const void* k, const void* v,
                       const float* sinks, const int32_t* cu_q, const int32_t* cu_k, int hq,
                       int hkv, float scale_log2, int causal, const StateSlots& ss, void* out,
                       float* lse, float* part_m, float* part_d, float* part_acc) {
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tv = static_cast<const T*>(v);
    T* to = static_cast<T*>(out);
    switch (lanes_per_pair(hq / hkv)) {
        case 4:
            hipLaunchKernelGGL((rows_kernel<T, kMode, 4>), grid, dim3(64), 0, stream, tq, tk, tv,
                               sinks, cu_q, cu_k, hq, hkv, scale_log2, causal, ss, to, lse, part_m,
                               part_d, part_acc);
            break;
        case 2:
            hipLaunchKernelGGL((rows_kernel<T, kMode, 2>), grid, dim3(64), 0, stream, tq, tk, tv,
                               sinks, cu_q, cu_k, hq, hkv, scale_log2, causal, ss, to, lse, part_m,
                               part_d, part_acc);
            break;
        default:
            hipLaunchKernelGGL((rows_kernel<T, kMode, 1>), grid, dim3(64), 0, stream, tq, tk, tv,
                               sinks, cu_q, cu_k, hq, hkv, scale_log2, causal, ss, to, lse, part_m,
                               part_d, part_acc);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_generic_prefill(bool bf16, const void* q, const void* k, const void* v,
                                  const float* sinks, const int32_t* cu_q, const int32_t* cu_k,
                                  int batch, int hq, int hkv, int max_lq, float sm_scale,
                                  int causal, void* out, float* lse, hipStream_t stream) {
    const int group = hq / hkv;
    const int rows_per_wave = 64 / (group * lanes_per_pair(group));
    const dim3 grid(ceil_div(max_lq, rows_per_wave), hkv, batch);
    const float sl = sm_scale * kLog2e;
    const StateSlots whole{0, 1, 1, 0, 1};
    return bf16 ? launch_rows<uint16_t, kRows>(grid, stream, q, k, v, sinks, cu_q, cu_k, hq, hkv, sl,
                                               causal, whole, out, lse, nullptr, nullptr, nullptr)
                : launch_rows<float, kRows>(grid, stream, q, k, v, sinks, cu_q, cu_k, hq, hkv, sl,
                                            causal, whole, out, lse, nullptr, nullptr, nullptr);
}

hipError_t launch_generic_decode_split(bool bf16, const void* q, const void* k, const void* v,
                                       const float* sinks, const int32_t* cu_k, int batch, int hq,
                                       int hkv, int chunk, int max_chunks, float sm_scale,
                                       float* part_m, float* part_d, float* part_acc,
                                       hipStream_t stream) {
    const dim3 grid(max_chunks, hkv, batch);
    const float sl = sm_scale * kLog2e;
    const StateSlots ss{chunk, max_chunks, max_chunks, 0, 1};
    return bf16 ? launch_rows<uint16_t, kDecodeSplit>(grid, stream, q, k, v, sinks, nullptr, cu_k, hq,
                                                      hkv, sl, 0, ss, nullptr, nullptr, part_m,
                                                      part_d, part_acc)
                : launch_rows<float, kDecodeSplit>(grid, stream, q, k, v, sinks, nullptr, cu_k, hq,
                                                   hkv, sl, 0, ss, nullptr, nullptr, part_m, part_d,
                                                   part_acc);
}

hipError_t launch_generic_prefill_split(bool bf16, const void* q, const void* k, const void* v,
                                        const float* sinks, const int32_t* cu_q,
                                        const int32_t* cu_k, int batch, int hq, int hkv,
                                        int max_lq, const StateSlots& ss, float sm_scale,
                                        int causal, float* part_m, float* part_d,
                                        float* part_acc, hipStream_t stream) {
    const int group = hq / hkv;
    const int rows_per_wave = 64 / (group * lanes_per_pair(group));
    const dim3 grid(ceil_div(max_lq, rows_per_wave), hkv, batch * ss.n_chunks);
    const float sl = sm_scale * kLog2e;
    return bf16 ? launch_rows<uint16_t, kRowsSplit>(grid, stream, q, k, v, sinks, cu_q, cu_k, hq, hkv,
                                                    sl, causal, ss, nullptr, nullptr, part_m,
                                                    part_d, part_acc)
                : launch_rows<float, kRowsSplit>(grid, stream, q, k, v, sinks, cu_q, cu_k, hq, hkv,
                                                 sl, causal, ss, nullptr, nullptr, part_m, part_d,
                                                 part_acc);
}

}  // namespace sa
