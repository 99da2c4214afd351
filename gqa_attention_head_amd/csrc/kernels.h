// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Where the split (state-writing) prefill kernels put their (m, d, acc) states:
// the keys of each sequence are cut into n_chunks chunks of `chunk` keys (one
// chunk per launch index); chunk c of query row r goes to slot r * stride + slot0
// + c of the [rows, Hq, stride] state buffers.  The head's sink enters chunk 0's
// state when `sink` is nonzero and no state otherwise.
struct StateSlots {
    int chunk;
    int n_chunks;
    int stride;
    int slot0;
    int sink;
};


// How a one-call decode cuts each sequence's keys into the blocks whose states the
// merge combines.  chunk > 0: fixed chunks, block c of sequence b = keys
// [c * chunk, min((c + 1) * chunk, L_b)).  chunk == 0: proportional blocks, the
// launch's `ranges` workgroups shared out so that every sequence gets one block
// plus a share of the other ranges - batch ones proportional to its keys
// (balanced_first_block); sequence b's n_b blocks split its keys evenly, block c
// = keys [c * C_b, min((c + 1) * C_b, L_b)) with C_b = ceil(L_b / n_b).  Either
// way a sequence has at most max_chunks blocks (the state slots per (sequence,
// head)).
struct DecodePlan {
    int chunk;
    int ranges;
    int max_seqlen_k;
    int max_chunks;
};

// Where the state of block c of sequence b, query head h sits in the state buffers:
// element b * seq + c * block + h * head of part_m / part_d (and that times head_dim
// in part_acc).  Chunk-major per head, [B, Hq, slots], for fixed chunks (the
// layout the ABI documents); block-major, [B, slots, Hq], for proportional blocks,
// so that one workgroup's states for all heads of a block are contiguous.
struct SlotLayout {
    int64_t seq, block, head;
};
__host__ __device__ inline SlotLayout head_major_slots(int hq, int slots) {
    return SlotLayout{(int64_t)hq * slots, 1, slots};
}
__host__ __device__ inline SlotLayout block_major_slots(int hq, int slots) {
    return SlotLayout{(int64_t)hq * slots, hq, 1};
}
__host__ __device__ inline SlotLayout plan_slots(const DecodePlan& p, int hq) {
    return p.chunk > 0 ? head_major_slots(hq, p.max_chunks) : block_major_slots(hq, p.max_chunks);
}

// Proportional blocks: how many of the ranges beyond one per sequence are shared
// out by key count, for a batch of `total` keys.  At most ranges - batch, and few
// enough that no sequence of up to max_seqlen_k keys gets more than max_chunks
// blocks (a sequence of L keys gets at most floor(L * extra / total) + 2).
__host__ __device__ inline int balanced_extra_blocks(int total, int batch, const DecodePlan& p) {
    if (total <= 0 || p.max_chunks < 2 || p.ranges <= batch) return 0;
    int64_t extra = p.ranges - batch;
    if (p.max_seqlen_k > 0) {
        const int64_t cap = (int64_t)(p.max_chunks - 2) * total / p.max_seqlen_k;
        extra = extra < cap ? extra : cap;
    }
    return (int)extra;
}

// Proportional blocks: the first block of sequence b, whose keys start `before`
// keys after the batch's first key: floor(before * extra / total) + b.  Strictly
// increasing in b, so every sequence gets at least one block; the batch has
// extra + batch blocks in all.
__host__ __device__ inline int balanced_first_block(int before, int b, int total, int extra) {
    return total > 0 ? (int)((int64_t)before * extra / total) + b : b;
}

// Vector-ALU kernel, float32 arithmetic; any group size G = hq / hkv <= 64, head_dim 64.
hipError_t launch_generic_prefill(bool bf16, const void* q, const void* k, const void* v,
                                  const float* sinks, const int32_t* cu_q, const int32_t* cu_k,
                                  int batch, int hq, int hkv, int max_lq, float sm_scale,
                                  int causal, void* out, float* lse, hipStream_t stream);
hipError_t launch_generic_prefill_split(bool bf16, const void* q, const void* k, const void* v,
                                        const float* sinks, const int32_t* cu_q,
                                        const int32_t* cu_k, int batch, int hq, int hkv,
                                        int max_lq, const StateSlots& ss, float sm_scale,
                                        int causal, float* part_m, float* part_d,
                                        float* part_acc, hipStream_t stream);
hipError_t launch_generic_decode_split(bool bf16, const void* q, const void* k, const void* v,
                                       const float* sinks, const int32_t* cu_k, int batch, int hq,
                                       int hkv, int chunk, int max_chunks, float sm_scale,
                                       float* part_m, float* part_d, float* part_acc,
                                       hipStream_t stream);

// bf16 matrix-core kernels, head_dim 64.
bool mfma_decode_supported(int group);
// Workgroups per key range of the matrix-core decode (blocks of eight waves, one
// wave per KV head or per slice of its query heads).
int mfma_decode_head_blocks(int hq, int hkv);
// Split pass of a one-call decode under `plan` (fixed chunks or proportional blocks).
hipError_t launch_mfma_decode_plan(const void* q, const void* k, const void* v,
                                   const float* sinks, const int32_t* cu_k, int batch, int hq,
                                   int hkv, const DecodePlan& plan, float sm_scale,
                                   float* part_m, float* part_d, float* part_acc,
                                   hipStream_t stream);
hipError_t launch_mfma_decode_split(const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_k, int batch, int hq,
                                    int hkv, int chunk, int max_chunks, float sm_scale,
                                    float* part_m, float* part_d, float* part_acc,
                                    hipStream_t stream);
bool mfma_prefill_supported(int group);
// max_lq and max_lk bound every sequence's query and key counts (grid sizing and
// work order).  Chunk states of every (query row, head, key chunk) instead of the output.
hipError_t launch_mfma_prefill_split(const void* q, const void* k, const void* v,
                                     const float* sinks, const int32_t* cu_q, const int32_t* cu_k,
                                     int batch, int hq, int hkv, int max_lq, int max_lk,
                                     const StateSlots& ss, float sm_scale, int causal,
                                     float* part_m, float* part_d, float* part_acc,
                                     hipStream_t stream);
hipError_t launch_mfma_prefill(const void* q, const void* k, const void* v, const float* sinks,
                               const int32_t* cu_q, const int32_t* cu_k, int batch, int hq,
                               int hkv, int max_lq, int max_lk, float sm_scale, int causal,
                               void* out, float* lse, hipStream_t stream);

// Top-K-then-softmax routing: bf16 logits [T, E], E in {8, ..., 512} (powers of
// two), 1 <= k <= 8; int32 indices and bf16 weights [T, k].
bool topk_softmax_supported(int num_experts);
hipError_t launch_topk_softmax(const void* logits, int64_t num_tokens, int num_experts, int k,
                               int32_t* indices, void* weights, hipStream_t stream);

// Bias add + rotary embedding of the fused QKV projection output (bf16, D = 64).
hipError_t launch_qkv_rope(const void* qkv, const void* bias, const int32_t* positions,
                           const float* cos_sin, int64_t num_tokens, int hq, int hkv, int rows,
                           void* q, void* k, void* v, hipStream_t stream);

// Log-sum-exp combination of split-KV chunk states.  cu_k == nullptr: every
// one of the max_chunks slots of each of the `batch` rows is combined.
hipError_t launch_merge(bool out_bf16, const float* part_m, const float* part_d,
                        const float* part_acc, const int32_t* cu_k, int chunk, int max_chunks,
                        int batch, int hq, void* out, float* lse, hipStream_t stream);
// The merge of a one-call decode under `plan`.
hipError_t launch_merge_plan(bool out_bf16, const float* part_m, const float* part_d,
                             const float* part_acc, const int32_t* cu_k, const DecodePlan& plan,
                             int batch, int hq, void* out, float* lse, hipStream_t stream);

// Bytes of the fixed per-device state array of sink_attn_decode_noalloc, and its
// address on the current device (looked up once per device, with it current).
constexpr size_t kDecodeScratchBytes = size_t(128) << 20;
hipError_t decode_scratch(float** ptr);

// One nontemporal 16-byte-load pass over `bytes` (a multiple of 16) of buf by
// num_blocks workgroups of 512 threads; out[block] = XOR of the 32-bit words the
// workgroup read.
hipError_t launch_read_probe(const void* buf, int64_t bytes, int num_blocks, uint32_t* out,
                             hipStream_t stream);

}  // namespace sa
