// Attention with a per-head sink over a packed varlen batch (prefill), bf16
// inputs, head_dim 64, matrix cores (gfx950).
//
// "GPT-OSS on day 0" (Perplexity), Kernels for GPT-OSS / Sink attention: the
// softmax is computed online with the maximum subtracted, the running maximum m
// starting at the head's sink and the running scale d at 1; the same kernel
// family serves prefill and decode.  The whole KV range of a query block is
// one block here, so the sink enters the state once, at the start.
//
// Work decomposition.  One workgroup per (sequence b, KV head g, group of 32-row
// query blocks); each wave handles one query head that shares KV head g
// (grouped-query attention) for one query block, so all of them share every K/V
// tile the workgroup stages in LDS.  Below eight heads per KV head a workgroup
// takes several consecutive query blocks; above sixteen the heads are cut into
// slices, one workgroup each.  Query blocks are issued heaviest first (the causal
// triangle gives late blocks the most keys).
//
// Per 64-key tile and wave (scores kept transposed, S^T = K Q^T, so that the
// exponentiated tile is already laid out as the B operand of the PV product):
//   S^T[64 keys x 32 rows] = K[64 x 64] . Q^T[64 x 32]      8 MFMA 32x32x16
//   bottom-right causal mask on diagonal tiles, online softmax in base 2 (the
//   row maximum is taken only when the running one is too low: see kSumLimit)
//   O^T[64 dims x 32 rows] += V^T[64 x 64] . P^T[64 x 32]   8 MFMA 32x32x16
//     (V read transposed out of LDS with ds_read_b64_tr_b16)
// K/V tiles are double-buffered: the next tile's global loads are in flight
// while the current tile is computed.
#include "common.h"
#include "decode_tile.h"
#include "kernels.h"

namespace sa {

namespace {

constexpr int kD = 64;
constexpr int kBQ = 32;             // query rows per wave
constexpr int kBK = 64;             // keys per tile
constexpr int kStride = kD + 8;     // LDS row stride of K tiles in bf16 elements (144 bytes)
// LDS row stride of V tiles (192 bytes): the transposed reads take 64 bytes of
// four consecutive rows per half-wave, which then fall in distinct banks.
constexpr int kVStride = kD + 32;
constexpr int kSegs = kBK * kD / 8; // 16-byte segments per K (or V) tile

// Exponentials are first taken against the running maximum m as it stands.  If a
// lane's sum of its 32 exponentials stays within kSumLimit, each of them does too
// (they are positive), the state needs no rescale and the tile skips the row-max
// reduction.  Otherwise (a score far above m, or an overflow) the tile takes its
// row maximum, rescales the state and exponentiates again.
constexpr float kSumLimit = 16384.0f;  // 2^14

// P^T tile in bf16, four 16-key slices (the B operand of O^T = V^T P^T): the
// exponentials 2^(s * scale_log2 - msub) of one lane's 32 scores; returns their
// fp32 sum (the lane's share of the running scale).  The scores are overwritten.
__device__ __forceinline__ float exp_tile(f32x16 (&s)[2], float scale_log2, float msub,
                                          bf16x8 (&pb)[4]) {
    // in place: arguments, then exponentials, then conversion and sum, so that no
    // instruction waits on the one just issued
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_fmaf(s[kb][i], scale_log2, -msub);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(s[kb][i]);
    __builtin_amdgcn_sched_barrier(0);
    float pair[16];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks / 2, hs = ks % 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = s[kb][8 * hs + 2 * e], p1 = s[kb][8 * hs + 2 * e + 1];
            const bf16x2 pk = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
            pb[ks][2 * e] = pk[0];
            pb[ks][2 * e + 1] = pk[1];
            pair[4 * ks + e] = p0 + p1;
        }
    }
#pragma unroll
    for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) pair[i] += pair[i + w];
    return pair[0];
}

// kSplit: the keys of each sequence are cut into ss.n_chunks chunks of ss.chunk
// keys, one chunk per launch index (the slowest grid dimension), and the kernel
// writes each row's state after its chunk (m in natural-log units, d, unnormalised
// acc) to slot (row, head, ss.slot0 + chunk) of buffers with ss.stride slots per
// (row, head), instead of the normalised output.  The sink enters chunk 0's state
// only, and only when ss.sink is set; a chunk a row cannot see leaves
// (m = -inf, d = 0, acc = 0).
// Consecutive 32-row query blocks per workgroup: the G query heads of a KV head for
// kQB blocks make G * kQB waves, which all share each K/V tile the workgroup stages.
// Up to 8 waves where G divides 8 (two workgroups per compute unit); below eight heads
// otherwise, up to 16 waves (G = 3, 5, 6, 7 leave 8-wave workgroups short of threads
// to stage a tile with one 16-byte load each, and the second load spilled registers).
constexpr int query_blocks(int G) { return G >= 8 ? 1 : (8 % G == 0 ? 8 / G : 16 / G); }

// A sequence with at most 16 / G query rows (decode steps, short chunks) in a
// workgroup of kWaves waves: up to eight waves split the keys of KV head g evenly,
// each streaming its share the way the split-KV decode does (decode_tile.h: nontemporal
// loads, two 32-key tiles in flight) for the L_q x G (row, head) columns, and the
// waves combine their states through LDS.  A 32-row query block per KV head would
// instead stream every key through one workgroup with one staged tile at a time.
// It reuses the tile buffers: waves 0-3 keep their V slices, then their state
// records, in the K buffers (lds_k), waves 4-7 in the V buffers (lds_v).
constexpr int kShortMaxCols = 16;
constexpr int kShortWaves = 8;
constexpr int kShortStateFloats = 2 * kShortMaxCols + kD * kShortMaxCols;  // m, d, acc
static_assert(4 * kDecodeVSlice <= 2 * kBK * kStride && 4 * kDecodeVSlice <= 2 * kBK * kVStride &&
                  4 * kShortStateFloats * 2 <= 2 * kBK * kStride,
              "four waves' V slices and state records fit in each pair of tile buffers");

template <int G, int kWaves>
__device__ __forceinline__ void short_rows(const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ sinks, int hq, int hkv,
                                           int g, int q0, int lq, int k0, int lk, int causal,
                                           float scale_log2, uint16_t* __restrict__ out,
                                           float* __restrict__ lse, uint16_t* lds_k,
                                           uint16_t* lds_v) {
    constexpr int nw = kWaves < kShortWaves ? kWaves : kShortWaves;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int q4 = lane / 16, c16 = lane % 16;
    // column c16 = (row r, head hh); columns past lq * G only pad the MFMA
    const bool col_ok = c16 < lq * G;
    const int r = col_ok ? c16 / G : 0, hh = c16 % G;
    const int h = g * G + hh;
    // keys row r sees (bottom-right causal alignment); the last row sees all lk
    const int lim = !col_ok ? 0 : causal ? max(0, min(lk, lk - lq + r + 1)) : lk;
    // this wave's share of the keys: equal runs of whole 32-key tiles
    const int per = ceil_div(ceil_div(lk, nw), kDecodeTileKeys) * kDecodeTileKeys;
    const int lo = min(wave * per, lk);
    const int hi = wave < nw ? min(lo + per, lk) : lo;

    WaveState st;
    st.m = (wave == 0 && col_ok) ? sinks[h] * kLog2e : kNegInf;  // the first block holds the sink
    st.dl = (q4 == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qb0 = {}, qb1 = {};
    if (col_ok) {
        const uint16_t* qp = q + ((int64_t)(q0 + r) * hq + h) * kD + 8 * q4;
        qb0 = load_bf16x8(qp);
        qb1 = load_bf16x8(qp + 32);
    }
    const int row_stride = hkv * kD;
    const uint16_t* kbase = k + ((int64_t)k0 * hkv + g) * kD;
    const uint16_t* vbase = v + ((int64_t)k0 * hkv + g) * kD;
    const int ws = wave < nw ? wave : 0;
    uint16_t* vw = (ws < 4 ? lds_k : lds_v) + (ws % 4) * kDecodeVSlice;
    const int ntiles = lo < hi ? ceil_div(hi - lo, kDecodeTileKeys) : 0;
    if (ntiles > 0) {  // (uniform per wave) see the split-KV decode's loop
        constexpr int kDepth = 2;
        DecodeTile buf[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            load_tile<true>(buf[d], kbase, vbase, row_stride, lo + d * kDecodeTileKeys, hi, lane);
        int it = 0;
        do {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int ts = lo + (it + d) * kDecodeTileKeys;
                process_tile(st, buf[d], qb0, qb1, vw, ts, min(lim, hi), scale_log2, lane);
                load_tile<true>(buf[d], kbase, vbase, row_stride, ts + kDepth * kDecodeTileKeys,
                                hi, lane);
            }
            it += kDepth;
        } while (it < ntiles);
    }
    st.dl += xor16(st.dl);
    st.dl = sum_xor32(st.dl);

    // combine: wave w's (m, d, acc) of every column into LDS, then one thread per
    // (column, dimension) output
    __syncthreads();  // every wave is done with its V slice
    auto record = [&](int w) {
        return reinterpret_cast<float*>(w < 4 ? lds_k : lds_v) + (w % 4) * kShortStateFloats;
    };
    if (wave < nw) {
        float* mine = record(wave);
        if (q4 == 0) {
            mine[c16] = st.m;
            mine[kShortMaxCols + c16] = st.dl;
        }
        float* acc = mine + 2 * kShortMaxCols;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[(16 * mt + 4 * q4 + i) * kShortMaxCols + c16] = st.o[mt][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < lq * G * kD; idx += 64 * kWaves) {
        const int col = idx / kD, dim = idx % kD;
        float big = kNegInf;
#pragma unroll
        for (int w = 0; w < nw; ++w) big = fmaxf(big, record(w)[col]);
        float num = 0.0f, den = 0.0f;
        if (big != kNegInf) {
#pragma unroll
            for (int w = 0; w < nw; ++w) {
                const float* st_w = record(w);
                const float mw = st_w[col];
                const float wt = mw == kNegInf ? 0.0f : fast_exp2(mw - big);
                den += wt * st_w[kShortMaxCols + col];
                num += wt * st_w[2 * kShortMaxCols + dim * kShortMaxCols + col];
            }
        }
        const bool empty = big == kNegInf || !(den > 0.0f);
        const int64_t orow = (int64_t)(q0 + col / G) * hq + g * G + col % G;
        out[orow * kD + dim] = f32_to_bf16_bits(empty ? 0.0f : num / den);
        if (lse != nullptr && dim == 0) lse[orow] = empty ? kNegInf : (big + fast_log2(den)) * kLn2;
    }
}

// kShortRows (unsplit launches whose keys outnumber their queries, G <= 16): the
// workgroups of sequences with at most 16 / G query rows take the short_rows path,
// and the first query group of every (sequence, KV head) pair is issued first.
template <int G, bool kSplit, bool kHeadSlices = false, bool kShortRows = false>
__global__ __launch_bounds__(64 * G * query_blocks(G)) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                  const uint16_t* __restrict__ v, const float* __restrict__ sinks,
                  const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int hq,
                  int hkv, int batch, int n_qgroups, int pair_major, float scale_log2, int causal,
                  uint16_t* __restrict__ out, float* __restrict__ lse, StateSlots ss,
                  float* __restrict__ part_m, float* __restrict__ part_d,
                  float* __restrict__ part_acc) {
    // kQB * G waves: the G query heads of KV head g for kQB consecutive query blocks
    constexpr int kQB = query_blocks(G);
    constexpr int kThreads = 64 * G * kQB;
    constexpr int kPer = (kSegs + kThreads - 1) / kThreads;
    __shared__ uint16_t kl[2][kBK * kStride];
    __shared__ uint16_t vl[2][kBK * kVStride];
    constexpr bool kShort = kShortRows && !kSplit && !kHeadSlices && G <= kShortMaxCols;

    // Work item -> (sequence b, KV head g, group of kQB query blocks qg).  Query
    // blocks go heaviest first (the causal triangle gives late blocks the most keys).
    // When the (b, g) pairs split evenly over the 8 XCDs (workgroups are dealt
    // to XCDs round-robin), each XCD keeps its own pairs, so a K/V head is
    // cached in one XCD's L2 only.  By default an XCD interleaves its pairs, one
    // query group of each in turn; pair_major (rows over longer key sets, such as
    // chunks over a cache) runs its pairs one after another instead, so that the
    // XCD streams the K/V of fewer heads at a time (measured faster there, slower
    // on equal query and key counts).
    // kHeadSlices: more than G query heads share KV head g; the group's
    // group / G slices of G heads each go to separate workgroups (slice hs slowest).
    const int pairs = batch * hkv;
    const int group = kHeadSlices ? hq / hkv : G;
    const int per_slice = pairs * n_qgroups;
    const int per_chunk = per_slice * (group / G);
    const int c = kSplit ? (int)(blockIdx.x / per_chunk) : 0;
    const int rest = kSplit ? (int)(blockIdx.x % per_chunk) : (int)blockIdx.x;
    const int hs = kHeadSlices ? rest / per_slice : 0;
    const int bid = kHeadSlices ? rest % per_slice : rest;
    // kShort: the first query group of every pair goes first (a pair of a decode
    // step or a short chunk has that one group only, and streams every key of its
    // sequence), then groups 1 .. n_qgroups - 1 as described.
    const int lead = kShort ? pairs : 0;
    const int ng = kShort ? max(n_qgroups - 1, 1) : n_qgroups;
    int pair, qg;
    if (kShort && bid < lead) {
        pair = bid;  // (pair % 8 == bid % 8: the XCD its other groups run on)
        qg = 0;
    } else if (pairs % 8 == 0) {
        const int rb = bid - lead;
        const int xcd = rb % 8, j = rb / 8, per_xcd = pairs / 8;
        pair = (pair_major ? j / ng : j % per_xcd) * 8 + xcd;
        qg = n_qgroups - 1 - (pair_major ? j % ng : j / per_xcd);
    } else {
        const int rb = bid - lead;
        pair = pair_major ? rb / ng : rb % pairs;
        qg = n_qgroups - 1 - (pair_major ? rb % ng : rb / pairs);
    }
    const int b = pair / hkv, g = pair % hkv;
    const int q0 = cu_q[b], lq = cu_q[b + 1] - q0;
    const int k0 = cu_k[b], lk = cu_k[b + 1] - k0;
    const int r0g = qg * kQB * kBQ;  // first row of the workgroup's query blocks
    if (r0g >= lq) return;           // uniform over the workgroup
    if constexpr (kShort) {
        if (lq * G <= kShortMaxCols) {  // uniform: a few query rows
            short_rows<G, G * kQB>(q, k, v, sinks, hq, hkv, g, q0, lq, k0, lk, causal, scale_log2,
                                   out, lse, &kl[0][0], &vl[0][0]);
            return;
        }
    }

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int h = g * group + hs * G + wave % G;
    const int r0 = r0g + (wave / G) * kBQ;  // this wave's query block
    const int l32 = lane % 32, half = lane / 32;
    const int row = r0 + l32;
    const bool row_ok = row < lq;
    const bool wave_live = r0 < lq;  // a wave past the last row only helps stage K/V
    const int last = min(r0 + kBQ, lq) - 1;
    const int last_wg = min(r0g + kQB * kBQ, lq) - 1;
    // keys [0, kend) are visible to some row of the wave's block, [0, kend_wg) to some
    // row of the workgroup, [0, full_end) to every row of the wave's block.
    int kend = causal ? max(0, min(lk, lk - lq + last + 1)) : lk;
    int kend_wg = causal ? max(0, min(lk, lk - lq + last_wg + 1)) : lk;
    int full_end = causal ? max(0, min(lk, lk - lq + r0 + 1)) : lk;
    // this launch's keys start at k_lo (0 unless split); rows see keys below row_lim
    const int k_lo = kSplit ? c * ss.chunk : 0;
    if (kSplit) {
        kend = min(kend, k_lo + ss.chunk);
        kend_wg = min(kend_wg, k_lo + ss.chunk);
        full_end = min(full_end, k_lo + ss.chunk);
    }
    const int row_lim = min(kend, causal ? lk - lq + row + 1 : lk);

    // B operand of S^T = K Q^T: lane holds Q[row][16*ks + 8*half .. +7].
    bf16x8 qop[4];
    {
        const uint16_t* qp = q + ((int64_t)(q0 + min(row, lq - 1)) * hq + h) * kD + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = load_bf16x8(qp + 16 * ks);
    }

    // Running state (base 2): the maximum starts at the sink (the first and only
    // block of keys holds it) and the scale at 1, split over the two lane halves.
    const bool with_sink = kSplit ? (c == 0 && ss.sink != 0) : true;
    float m = with_sink ? sinks[h] * kLog2e : kNegInf;
    float dl = (half == 0 && with_sink) ? 1.0f : 0.0f;
    f32x16 o[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mt][i] = 0.0f;

    const int row_stride = hkv * kD;
    const uint16_t* kbase = k + ((int64_t)k0 * hkv + g) * kD;
    const uint16_t* vbase = v + ((int64_t)k0 * hkv + g) * kD;
    u32x4 kreg[kPer], vreg[kPer];
    auto gload = [&](int j0) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int idx = threadIdx.x + p * kThreads;
            if (kSegs % kThreads == 0 || idx < kSegs) {
                const int key = min(j0 + idx / 8, lk - 1);
                const int64_t off = (int64_t)key * row_stride + 8 * (idx % 8);
                kreg[p] = *reinterpret_cast<const u32x4*>(kbase + off);
                vreg[p] = *reinterpret_cast<const u32x4*>(vbase + off);
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int idx = threadIdx.x + p * kThreads;
            if (kSegs % kThreads == 0 || idx < kSegs) {
                *reinterpret_cast<u32x4*>(&kl[buf][(idx / 8) * kStride + 8 * (idx % 8)]) = kreg[p];
                *reinterpret_cast<u32x4*>(&vl[buf][(idx / 8) * kVStride + 8 * (idx % 8)]) = vreg[p];
            }
        }
    };

    // 64-key tiles t_first .. ntiles - 1 cover [k_lo, kend_wg)
    const int t_first = k_lo / kBK;
    const int ntiles = (kend_wg > k_lo) ? ceil_div(kend_wg, kBK) : t_first;
    if (ntiles > t_first) {
        gload(t_first * kBK);
        lstore(t_first & 1);
    }
    __syncthreads();
    const int g4 = lane / 16, c16 = lane % 16;
    for (int t = t_first; t < ntiles; ++t) {
        const int j0 = t * kBK;
        const int buf = t & 1;
        const bool more = t + 1 < ntiles;
        if (more) gload(j0 + kBK);
        const uint16_t* kt = kl[buf];
        const uint16_t* vt = vl[buf];

        // raw scores: s[kb][i] = <q_row, k_key>, key = j0 + 32*kb + 8*(i/4) + 4*half + i%4,
        // keys outside [k_lo, row_lim) masked to -inf on an edge tile (diagonal, ragged
        // or chunk edge; uniform).  A macro rather than a function: this kernel sits at
        // the 128-VGPR limit, and the function form made the compiler spill.
#define SA_SCORES()                                                                              \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                           \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;                          \
        _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) {                                       \
            const bf16x8 a = load_bf16x8(kt + (32 * kb + l32) * kStride + 16 * ks + 8 * half);   \
            s[kb] = mfma32x32x16(a, qop[ks], s[kb]);                                             \
        }                                                                                        \
    }                                                                                            \
    if (j0 + kBK > full_end || j0 < k_lo) {                                                      \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                         \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                         \
            const int key = j0 + 32 * kb + 8 * (i / 4) + 4 * half + (i % 4);                     \
            if (key >= row_lim || key < k_lo) s[kb][i] = kNegInf;                                \
        }                                                                                        \
    }
        // a wave whose block sees none of this tile's keys only helps stage K/V
        // (uniform per wave; always true with one query block per workgroup)
        if (kQB == 1 || (wave_live && j0 < kend)) {
            f32x16 s[2];
            SA_SCORES()
            bf16x8 pb[4];
            float psum;
            // no finite reference yet (no sink and no visible key so far): take the max
            bool need_max = __any(m == kNegInf);
            if (!need_max) {
                psum = exp_tile(s, scale_log2, m, pb);
                need_max = __any(!(psum <= kSumLimit));
            }
            if (need_max) {  // rare: recompute the scores rather than keep them live
                SA_SCORES()
                float tmax = kNegInf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]);
                const float m_new = fmaxf(m, max_xor32(tmax) * scale_log2);
                const float alpha = (m == kNegInf) ? 0.0f : fast_exp2(m - m_new);
                dl *= alpha;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) o[mt] *= alpha;
                m = m_new;
                const float msub = (m == kNegInf) ? 0.0f : m;
                psum = exp_tile(s, scale_log2, msub, pb);
            }
#undef SA_SCORES
            dl += psum;

#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int key_base = 32 * (ks / 2) + 16 * (ks % 2);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const uint16_t* p0 = vt + (key_base + 4 * half + c16 / 4) * kVStride + 32 * mt +
                                         16 * (g4 % 2) + 4 * (c16 % 4);
                    const bf16x8 va = concat(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * kVStride));
                    o[mt] = mfma32x32x16(va, pb[ks], o[mt]);
                }
            }
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
    }

    const float dsum = sum_xor32(dl);
    if (!row_ok) return;
    const int64_t orow = (int64_t)(q0 + row) * hq + h;
    if (kSplit) {
        const int64_t slot = orow * ss.stride + ss.slot0 + c;
        float* pa = part_acc + slot * kD;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                // o[mt][4j + e] = O^T[dim 32*mt + 8*j + 4*half + e][row]
                *reinterpret_cast<f32x4*>(pa + 32 * mt + 8 * j + 4 * half) =
                    f32x4{o[mt][4 * j], o[mt][4 * j + 1], o[mt][4 * j + 2], o[mt][4 * j + 3]};
        if (half == 0) {
            part_m[slot] = (m == kNegInf) ? kNegInf : m * kLn2;
            part_d[slot] = dsum;
        }
        return;
    }
    const bool empty = (m == kNegInf) || !(dsum > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / dsum;
    uint16_t* op = out + orow * kD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // o[mt][4j + e] = O^T[dim 32*mt + 8*j + 4*half + e][row]
            const bf16x2 lo2 = __builtin_convertvector(
                f32x2{o[mt][4 * j + 0] * inv, o[mt][4 * j + 1] * inv}, bf16x2);
            const bf16x2 hi2 = __builtin_convertvector(
                f32x2{o[mt][4 * j + 2] * inv, o[mt][4 * j + 3] * inv}, bf16x2);
            *reinterpret_cast<u32x2*>(op + 32 * mt + 8 * j + 4 * half) =
                u32x2{__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)};
        }
    if (lse != nullptr && half == 0)
        lse[orow] = empty ? kNegInf : (m + fast_log2(dsum)) * kLn2;
}

template <int G, bool kHeadSlices>
hipError_t launch_g(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_q, const int32_t* cu_k, int batch, int hq, int hkv,
                    int max_lq, int max_lk, float sm_scale, int causal, void* out, float* lse,
                    const StateSlots& ss, float* part_m, float* part_d, float* part_acc,
                    hipStream_t stream) {
    constexpr int kQB = query_blocks(G);  // query blocks per workgroup
    const int n_qgroups = ceil_div(ceil_div(max_lq, kBQ), kQB);
    const int pair_major = max_lk > max_lq;
    const int slices = (hq / hkv) / G;      // workgroups per (sequence, KV head, block group)
    const bool split = part_m != nullptr;
    const int64_t blocks =
        (int64_t)batch * hkv * n_qgroups * slices * (split ? ss.n_chunks : 1);
    const dim3 threads(64 * G * kQB);
    if (split)
        hipLaunchKernelGGL((prefill_mfma<G, true, kHeadSlices>), dim3((unsigned)blocks), threads, 0,
                           stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           sinks, cu_q, cu_k, hq, hkv, batch, n_qgroups, pair_major, sm_scale * kLog2e, causal,
                           nullptr, nullptr, ss, part_m, part_d, part_acc);
    else if (!kHeadSlices && G <= kShortMaxCols && pair_major)
        hipLaunchKernelGGL((prefill_mfma<G, false, false, true>), dim3((unsigned)blocks), threads, 0,
                           stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           sinks, cu_q, cu_k, hq, hkv, batch, n_qgroups, pair_major, sm_scale * kLog2e, causal,
                           (uint16_t*)out, lse, ss, nullptr, nullptr, nullptr);
    else
        hipLaunchKernelGGL((prefill_mfma<G, false, kHeadSlices>), dim3((unsigned)blocks), threads, 0,
                           stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                           sinks, cu_q, cu_k, hq, hkv, batch, n_qgroups, pair_major, sm_scale * kLog2e, causal,
                           (uint16_t*)out, lse, ss, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t dispatch(const void* q, const void* k, const void* v, const float* sinks,
                    const int32_t* cu_q, const int32_t* cu_k, int batch, int hq, int hkv,
                    int max_lq, int max_lk, float sm_scale, int causal, void* out, float* lse,
                    const StateSlots& ss, float* part_m, float* part_d, float* part_acc,
                    hipStream_t stream) {
    const int group = hq / hkv;
#define SA_ARGS q, k, v, sinks, cu_q, cu_k, batch, hq, hkv, max_lq, max_lk, sm_scale, causal, out, lse, ss, part_m, part_d, part_acc, stream
    switch (group) {
#define SA_CASE(GG) case GG: return launch_g<GG, false>(SA_ARGS);
        SA_CASE(1) SA_CASE(2) SA_CASE(3) SA_CASE(4) SA_CASE(5) SA_CASE(6) SA_CASE(7) SA_CASE(8)
        SA_CASE(9) SA_CASE(10) SA_CASE(11) SA_CASE(12) SA_CASE(13) SA_CASE(14) SA_CASE(15) SA_CASE(16)
#undef SA_CASE
        default: break;
    }
    // more than 16 heads per KV head: slices of the largest power of two <= 16 that
    // divides the group
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

}  // namespace

hipError_t launch_mfma_prefill(const void* q, const void* k, const void* v, const float* sinks,
                               const int32_t* cu_q, const int32_t* cu_k, int batch, int hq,
                               int hkv, int max_lq, int max_lk, float sm_scale, int causal,
                               void* out, float* lse, hipStream_t stream) {
    const StateSlots whole{0, 1, 1, 0, 1};  // one block of keys, sink included
    return dispatch(q, k, v, sinks, cu_q, cu_k, batch, hq, hkv, max_lq, max_lk, sm_scale, causal,
                    out, lse, whole, nullptr, nullptr, nullptr, stream);
}

hipError_t launch_mfma_prefill_split(const void* q, const void* k, const void* v,
                                     const float* sinks, const int32_t* cu_q, const int32_t* cu_k,
                                     int batch, int hq, int hkv, int max_lq, int max_lk,
                                     const StateSlots& ss, float sm_scale, int causal,
                                     float* part_m, float* part_d, float* part_acc,
                                     hipStream_t stream) {
    return dispatch(q, k, v, sinks, cu_q, cu_k, batch, hq, hkv, max_lq, max_lk, sm_scale, causal,
                    nullptr, nullptr, ss, part_m, part_d, part_acc, stream);
}

}  // namespace sa
