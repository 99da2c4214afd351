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
#include "decode_tile.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kTile = kDecodeTileKeys;
constexpr int kVStride = kDecodeVStride;

// The query heads one wave serves: KV head g and, above 16 query heads per KV
// head, slice hs of G of them (one wave per slice); lane (q4, c16) holds head
// column c16, which is query head h.
struct WaveHeads {
    int g, h;
    bool g_ok, head_ok;
};

template <int G, bool kHeadSlices>
__device__ __forceinline__ WaveHeads wave_heads(int hq, int hkv, int hb, int heads_per_block,
                                                int wave, int lane) {
    const int group = kHeadSlices ? hq / hkv : G;
    const int slices = group / G;
    const int u = hb * heads_per_block + wave;
    WaveHeads w;
    w.g = kHeadSlices ? u / slices : u;
    const int hs = kHeadSlices ? u % slices : 0;
    w.g_ok = w.g < hkv;
    w.head_ok = w.g_ok && (lane % 16) < G;
    w.h = w.g * group + hs * G + lane % 16;
    return w;
}

// State of the wave's query heads after keys [lo, hi) of sequence b (indices
// within the sequence, whose key 0 is row k0 of k and v), written to slot c of
// the (b, h) state buffers; the running maximum starts at the head's sink when
// with_sink (the block that holds the sequence's first key), else at -inf.
template <int G, int kDepth, bool kHeadSlices>
__device__ __forceinline__ void run_range(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks, const WaveHeads& wh,
    int hq, int hkv, int b, int k0, int lo, int hi, bool with_sink, int c, SlotLayout slots,
    float scale_log2, uint16_t* vw, int lane, float* __restrict__ part_m,
    float* __restrict__ part_d, float* __restrict__ part_acc) {
    const int q4 = lane / 16;
    const int row_stride = hkv * kD;
    const int gsafe = wh.g_ok ? wh.g : 0;
    const uint16_t* kbase = k + ((int64_t)k0 * hkv + gsafe) * kD;
    const uint16_t* vbase = v + ((int64_t)k0 * hkv + gsafe) * kD;

    // the scale starts at 1, held by one lane share (q4 == 0)
    WaveState st;
    st.m = (with_sink && wh.head_ok) ? sinks[wh.h] * kLog2e : kNegInf;
    st.dl = (q4 == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (wh.g_ok && lo < hi) ? ceil_div(hi - lo, kTile) : 0;
    // B operand of S^T = K Q^T: lane holds Q[head c16][dims 8*q4 .. +7] (and +32).
    bf16x8 qb0 = {}, qb1 = {};
    if (wh.head_ok) {
        const uint16_t* qp = q + ((int64_t)b * hq + wh.h) * kD + 8 * q4;
        qb0 = load_bf16x8(qp);
        qb1 = load_bf16x8(qp + 32);
    }

    // kDepth tiles of loads stay in flight per wave.  Loads are issued
    // unconditionally (addresses clamped to the range's last key, which exists
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
    const int64_t slot = b * slots.seq + c * slots.block + wh.h * slots.head;
    if (wh.head_ok) {
        float* pa = part_acc + slot * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(pa + 16 * mt + 4 * q4) = st.o[mt];
        if (q4 == 0) {
            part_m[slot] = m_nat;
            part_d[slot] = st.dl;
        }
    }
}

// Fixed chunks: one workgroup per (sequence b, chunk c, block of KV heads).
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
    const WaveHeads wh = wave_heads<G, kHeadSlices>(hq, hkv, hb, kHeadsPerBlock, wave, lane);
    // m starts at the sink in chunk 0 only
    run_range<G, kDepth, kHeadSlices>(q, k, v, sinks, wh, hq, hkv, b, k0, lo, hi, c == 0, c,
                                      head_major_slots(hq, max_chunks), scale_log2, vlds[wave],
                                      lane, part_m, part_d, part_acc);
}

// Proportional blocks: the sequence b that workgroup w serves, the largest b with
// balanced_first_block(b) <= w (block 0 is sequence 0's, and the first blocks
// increase strictly, so it exists for every w below the batch's block count).  The
// wave probes up to 64 sequences at a time, narrowing the range 64-fold per round
// (one round for up to 64 sequences); clamped into [0, batch) whatever the offsets
// hold.
__device__ __forceinline__ int find_block(const int32_t* __restrict__ cu_k, int batch, int base,
                                          int total, int extra, int w, int lane) {
    // p* = the first sequence p in [1, batch] whose first block lies past w (p = batch
    // always does); the answer is p* - 1.  p* lies in [lo, lo + n).
    int lo = 1, n = batch;
    while (n > 1) {
        const int step = ceil_div(n, 64);
        const bool probe = lane * step < n;
        const int p = min(lo + lane * step, batch);
        const bool past = probe && balanced_first_block(cu_k[p] - base, p, total, extra) > w;
        const uint64_t hits = __ballot(past);
        if (hits != 0) {
            // p* lies after the last probe that is not past w, up to the first that is
            const int f = __builtin_ctzll(hits);
            const int nlo = f == 0 ? lo : lo + (f - 1) * step + 1;
            n = lo + f * step - nlo + 1;
            lo = nlo;
        } else {
            const int top = 63 - __builtin_clzll(__ballot(probe));
            const int nlo = lo + top * step + 1;
            n = lo + n - nlo;
            lo = nlo;
        }
    }
    return max(0, min(lo - 1, batch - 1));
}

// Proportional blocks (see DecodePlan): workgroup column w serves block c of one
// sequence, c = w - (first block of that sequence), so that every compute unit
// streams about the same number of bytes and no workgroup crosses a sequence.
template <int G, int kDepth, int kHeadsPerBlock, bool kHeadSlices = false>
__global__ __launch_bounds__(64 * kHeadsPerBlock) void decode_balanced_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_k, int batch, int hq, int hkv, DecodePlan plan,
    int head_blocks, float scale_log2, float* __restrict__ part_m,
    float* __restrict__ part_d, float* __restrict__ part_acc) {
    __shared__ uint16_t vlds[kHeadsPerBlock][kTile * kVStride];

    const int hb = blockIdx.x % head_blocks;
    const int w = blockIdx.x / head_blocks;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    // Up to 64 sequences: lane l reads the end offset of sequence l together with the
    // batch's first and last offsets (one round trip gives the sequence and its keys).
    const int ends = (batch <= 64 && lane < batch) ? cu_k[lane + 1] : 0;
    const int base = cu_k[0];
    const int total = cu_k[batch] - base;
    const int extra = balanced_extra_blocks(total, batch, plan);
    if (w >= extra + batch) return;  // uniform: the batch has fewer blocks

    int b, k0, k1;
    if (batch <= 64) {
        // b = the first sequence whose successor's first block lies past w
        const uint64_t past = __ballot(lane < batch &&
                                       balanced_first_block(ends - base, lane + 1, total, extra) > w);
        b = past != 0 ? __builtin_ctzll(past) : batch - 1;
        k0 = b == 0 ? base : __builtin_amdgcn_readlane(ends, b - 1);
        k1 = __builtin_amdgcn_readlane(ends, b);
    } else {
        b = __builtin_amdgcn_readfirstlane(find_block(cu_k, batch, base, total, extra, w, lane));
        k0 = cu_k[b];
        k1 = cu_k[b + 1];
    }
    const int first = balanced_first_block(k0 - base, b, total, extra);
    const int nblk = balanced_first_block(k1 - base, b + 1, total, extra) - first;
    const int c = w - first;
    const int per = ceil_div(max(k1 - k0, 0), max(nblk, 1));
    const int len = max(k1 - k0, 0);
    if (c < 0 || c >= plan.max_chunks) return;  // only with broken offsets
    const int lo = min(c * per, len);  // (an empty block holds the empty state)
    const int hi = min(lo + per, len);
    const WaveHeads wh = wave_heads<G, kHeadSlices>(hq, hkv, hb, kHeadsPerBlock, wave, lane);
    run_range<G, kDepth, kHeadSlices>(q, k, v, sinks, wh, hq, hkv, b, k0, lo, hi, c == 0, c,
                                      block_major_slots(hq, plan.max_chunks), scale_log2,
                                      vlds[wave], lane, part_m, part_d, part_acc);
}

template <int G, bool kHeadSlices>
hipError_t launch_g(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_k, int batch, int hq, int hkv, const DecodePlan& plan,
                    float sm_scale, float* part_m, float* part_d, float* part_acc,
                    hipStream_t stream) {
    constexpr int kDepth = 2, kHeadsPerBlock = 8;
    const int units = hkv * ((hq / hkv) / G);  // (KV head, slice of G query heads)
    const int head_blocks = ceil_div(units, kHeadsPerBlock);
    if (plan.chunk > 0) {
        const int64_t blocks = (int64_t)batch * plan.max_chunks * head_blocks;
        hipLaunchKernelGGL((decode_split_mfma<G, kDepth, kHeadsPerBlock, kHeadSlices>),
                           dim3((unsigned)blocks), dim3(64 * kHeadsPerBlock), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks,
                           cu_k, hq, hkv, plan.chunk, plan.max_chunks, head_blocks,
                           sm_scale * kLog2e, part_m, part_d, part_acc);
    } else {
        const int64_t blocks = (int64_t)plan.ranges * head_blocks;
        hipLaunchKernelGGL((decode_balanced_mfma<G, kDepth, kHeadsPerBlock, kHeadSlices>),
                           dim3((unsigned)blocks), dim3(64 * kHeadsPerBlock), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, sinks,
                           cu_k, batch, hq, hkv, plan, head_blocks, sm_scale * kLog2e, part_m,
                           part_d, part_acc);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_decode_plan(const void* q, const void* k, const void* v,
                                   const float* sinks, const int32_t* cu_k, int batch, int hq,
                                   int hkv, const DecodePlan& plan, float sm_scale,
                                   float* part_m, float* part_d, float* part_acc,
                                   hipStream_t stream) {
    const int group = hq / hkv;
#define SA_ARGS q, k, v, sinks, cu_k, batch, hq, hkv, plan, sm_scale, part_m, part_d, part_acc, stream
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

hipError_t launch_mfma_decode_split(const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_k, int batch, int hq,
                                    int hkv, int chunk, int max_chunks, float sm_scale,
                                    float* part_m, float* part_d, float* part_acc,
                                    hipStream_t stream) {
    const DecodePlan plan{chunk, 0, 0, max_chunks};
    return launch_mfma_decode_plan(q, k, v, sinks, cu_k, batch, hq, hkv, plan, sm_scale, part_m,
                                   part_d, part_acc, stream);
}

}  // namespace sa
