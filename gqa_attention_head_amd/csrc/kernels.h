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

// One nontemporal 16-byte-load pass over `bytes` (a multiple of 16) of buf by
// num_blocks workgroups of 512 threads; out[block] = XOR of the 32-bit words the
// workgroup read.
hipError_t launch_read_probe(const void* buf, int64_t bytes, int num_blocks, uint32_t* out,
                             hipStream_t stream);

}  // namespace sa
