// C ABI of the library: argument validation, kernel selection and launch.
// Every check that needs only host data happens before anything is launched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <string>
#include <vector>

#include "kernels.h"
#include "moe_router.h"
#include "qkv_epilogue.h"
#include "sa_measure.h"
#include "sink_attn.h"

static_assert(SA_DECODE_SCRATCH_BYTES == sa::kDecodeScratchBytes,
              "the header states the size of the decode state array");

namespace {

thread_local std::string g_last_error;

sa_status_t fail(sa_status_t status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

sa_status_t ok() {
    g_last_error.clear();
    return SA_OK;
}

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("SINK_ATTN_DEBUG");
        return e != nullptr && e[0] == '1';
    }();
    return on;
}

sa_status_t check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SA_ELAUNCH, "no HIP device available: %s", hipGetErrorString(e));
    }
    return SA_OK;
}

sa_status_t finish_launch(hipError_t e, hipStream_t stream, const char* what) {
    if (e != hipSuccess) return fail(SA_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    if (debug_sync()) {
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return fail(SA_ELAUNCH, "%s: kernel failed: %s", what, hipGetErrorString(e));
    }
    return ok();
}

sa_status_t check_heads(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim) {
    if (batch < 1 || batch > 65535) return fail(SA_EINVAL, "batch must be in [1, 65535], got %d", batch);
    if (hq < 1 || hkv < 1) return fail(SA_EINVAL, "head counts must be >= 1 (Hq=%d, Hkv=%d)", hq, hkv);
    if (hq % hkv != 0) return fail(SA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", hq, hkv);
    if (hkv > 65535) return fail(SA_EINVAL, "Hkv must be <= 65535, got %d", hkv);
    if (hq / hkv > 64) return fail(SA_EUNSUPPORTED, "group size Hq/Hkv = %d > 64 is not supported", hq / hkv);
    if (head_dim != 64) return fail(SA_EUNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
    return SA_OK;
}

// With SINK_ATTN_DEBUG=1, the preconditions that live in device memory are checked
// too, at the cost of a synchronisation: sequence offsets nondecreasing, lengths
// within the max_seqlen_* bounds, L_q <= L_k under causal masking, sinks neither
// +inf nor NaN.  cu_q == nullptr means one query per sequence (decode).
sa_status_t debug_check_inputs(hipStream_t stream, const int32_t* cu_q, const int32_t* cu_k,
                               int32_t batch, int32_t max_q, int32_t max_k, int32_t causal,
                               const float* sinks, int32_t hq) {
    if (!debug_sync()) return SA_OK;
    hipError_t e = hipStreamSynchronize(stream);
    std::vector<int32_t> hq_cu(batch + 1, 0), hk_cu(batch + 1, 0);
    std::vector<float> hs(sinks ? hq : 0);
    if (e == hipSuccess && cu_q)
        e = hipMemcpy(hq_cu.data(), cu_q, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost);
    if (e == hipSuccess && cu_k)
        e = hipMemcpy(hk_cu.data(), cu_k, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost);
    if (e == hipSuccess && sinks)
        e = hipMemcpy(hs.data(), sinks, sizeof(float) * hq, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(SA_ELAUNCH, "debug input check: %s", hipGetErrorString(e));
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t lk = (int64_t)hk_cu[b + 1] - hk_cu[b];
        const int64_t lq = cu_q ? (int64_t)hq_cu[b + 1] - hq_cu[b] : 1;
        if (lk < 0 || lq < 0)
            return fail(SA_EINVAL, "debug: cu_seqlens decrease at sequence %d", b);
        if (lk > max_k) return fail(SA_EINVAL, "debug: sequence %d has %lld keys > max_seqlen_k %d", b, (long long)lk, max_k);
        if (cu_q && lq > max_q) return fail(SA_EINVAL, "debug: sequence %d has %lld queries > max_seqlen_q %d", b, (long long)lq, max_q);
        if (cu_q && causal && lq > lk) return fail(SA_EINVAL, "debug: sequence %d has L_q %lld > L_k %lld under causal masking", b, (long long)lq, (long long)lk);
    }
    for (int32_t h = 0; h < (int32_t)hs.size(); ++h)
        if (std::isnan(hs[h]) || hs[h] == INFINITY)
            return fail(SA_EINVAL, "debug: sink of head %d is %f (must be finite or -inf)", h, hs[h]);
    return SA_OK;
}

// Bound on the query blocks the MFMA prefill launches cover: its workgroups group
// up to 16 consecutive blocks, so the count is rounded up by less than 16.
int64_t qblocks_bound(int32_t max_seqlen_q) { return (int64_t)(max_seqlen_q + 31) / 32 + 15; }

// A launch's x dimension counts work-items in 32 bits: blocks * threads per block
// must stay below 2^32.
sa_status_t check_grid(int64_t blocks, int64_t threads_per_block, const char* what) {
    if (blocks > 0 && blocks > (int64_t)0xFFFFFFFFLL / threads_per_block)
        return fail(SA_EINVAL, "%s: %lld blocks of %lld threads exceed the 2^32 work-item grid limit",
                    what, (long long)blocks, (long long)threads_per_block);
    return SA_OK;
}

// Chunk c covers keys [c * C, (c + 1) * C); the kernels form these bounds in 32 bits
// for every c < max_num_chunks, so max_num_chunks * C must stay below 2^31.
sa_status_t check_chunk_span(int32_t kv_chunk_size, int32_t max_num_chunks, const char* what) {
    if ((int64_t)kv_chunk_size * max_num_chunks > (int64_t)INT32_MAX)
        return fail(SA_EINVAL, "%s: max_num_chunks (%d) * kv_chunk_size (%d) exceeds 2^31 - 1",
                    what, max_num_chunks, kv_chunk_size);
    return SA_OK;
}

// The kernels move q, k, v and the accumulator states in 16-byte pieces and a prefill
// output row in 8-byte pieces: those pointers must be aligned to match.
bool aligned(const void* p, uintptr_t bytes) {
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}
sa_status_t check_alignment(const char* what, const void* q, const void* k, const void* v,
                            const void* part_acc, const void* out, uintptr_t out_bytes) {
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(part_acc, 16))
        return fail(SA_EINVAL, "%s: q, k, v and part_acc must be 16-byte aligned", what);
    if (!aligned(out, out_bytes))
        return fail(SA_EINVAL, "%s: out must be %u-byte aligned", what, (unsigned)out_bytes);
    return SA_OK;
}

sa_status_t check_dtype(sa_dtype_t d) {
    if (d != SA_FP32 && d != SA_BF16) return fail(SA_EINVAL, "unknown dtype %d", (int)d);
    return SA_OK;
}

}  // namespace

extern "C" {

const char* sink_attn_last_error(void) { return g_last_error.c_str(); }

sa_status_t sink_attn_prefill(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                              const float* sinks, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, float sm_scale, int32_t causal, void* out,
                              float* lse, void* stream) {
    sa_status_t s;
    if ((s = check_dtype(dtype)) != SA_OK) return s;
    if (!q || !k || !v || !sinks || !cu_seqlens_q || !cu_seqlens_k || !out)
        return fail(SA_EINVAL, "sink_attn_prefill: null pointer argument");
    if ((s = check_alignment("sink_attn_prefill", q, k, v, nullptr, out, 8)) != SA_OK) return s;
    if ((s = check_heads(batch, num_q_heads, num_kv_heads, head_dim)) != SA_OK) return s;
    if (max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(SA_EINVAL, "max_seqlen_q/max_seqlen_k must be >= 0");
    if (causal != 0 && causal != 1) return fail(SA_EINVAL, "causal must be 0 or 1");
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SA_EINVAL, "sm_scale must be finite and > 0");
    const int group = num_q_heads / num_kv_heads;
    const bool mfma = dtype == SA_BF16 && sa::mfma_prefill_supported(group);
    if (mfma && (s = check_grid((int64_t)batch * num_kv_heads * qblocks_bound(max_seqlen_q),
                                64 * group, "sink_attn_prefill")) != SA_OK)
        return s;
    if (!mfma && (s = check_grid(max_seqlen_q, 64, "sink_attn_prefill")) != SA_OK) return s;
    if (max_seqlen_q == 0) return ok();
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, causal, sinks, num_q_heads)) != SA_OK) return s;
    hipError_t e;
    if (mfma)
        e = sa::launch_mfma_prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, batch, num_q_heads,
                                    num_kv_heads, max_seqlen_q, max_seqlen_k, sm_scale, causal, out,
                                    lse, st);
    else
        e = sa::launch_generic_prefill(dtype == SA_BF16, q, k, v, sinks, cu_seqlens_q,
                                       cu_seqlens_k, batch, num_q_heads, num_kv_heads,
                                       max_seqlen_q, sm_scale, causal, out, lse, st);
    return finish_launch(e, st, "sink_attn_prefill");
}

sa_status_t sink_attn_prefill_split(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t kv_chunk_size, int32_t max_num_chunks, float sm_scale,
                                    int32_t causal, float* part_m, float* part_d, float* part_acc,
                                    void* stream) {
    sa_status_t s;
    if ((s = check_dtype(dtype)) != SA_OK) return s;
    if (!q || !k || !v || !sinks || !cu_seqlens_q || !cu_seqlens_k || !part_m || !part_d ||
        !part_acc)
        return fail(SA_EINVAL, "sink_attn_prefill_split: null pointer argument");
    if ((s = check_alignment("sink_attn_prefill_split", q, k, v, part_acc, nullptr, 1)) != SA_OK)
        return s;
    if ((s = check_heads(batch, num_q_heads, num_kv_heads, head_dim)) != SA_OK) return s;
    if (max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(SA_EINVAL, "max_seqlen_q/max_seqlen_k must be >= 0");
    if (causal != 0 && causal != 1) return fail(SA_EINVAL, "causal must be 0 or 1");
    if (kv_chunk_size < 1) return fail(SA_EINVAL, "kv_chunk_size must be >= 1, got %d", kv_chunk_size);
    const int64_t need = max_seqlen_k == 0 ? 1 : ((int64_t)max_seqlen_k + kv_chunk_size - 1) / kv_chunk_size;
    if (max_num_chunks < need)
        return fail(SA_EINVAL, "max_num_chunks (%d) < ceil(max_seqlen_k / kv_chunk_size) = %lld",
                    max_num_chunks, (long long)need);
    if ((s = check_chunk_span(kv_chunk_size, max_num_chunks, "sink_attn_prefill_split")) != SA_OK)
        return s;
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SA_EINVAL, "sm_scale must be finite and > 0");
    const int group = num_q_heads / num_kv_heads;
    const bool mfma = dtype == SA_BF16 && sa::mfma_prefill_supported(group);
    if (mfma) {
        if ((s = check_grid((int64_t)batch * num_kv_heads * qblocks_bound(max_seqlen_q) * max_num_chunks,
                            64 * group, "sink_attn_prefill_split")) != SA_OK)
            return s;
    } else if ((int64_t)batch * max_num_chunks > 65535) {
        return fail(SA_EINVAL, "batch * max_num_chunks must be <= 65535 on this path");
    } else if ((s = check_grid(max_seqlen_q, 64, "sink_attn_prefill_split")) != SA_OK) {
        return s;
    }
    if (max_seqlen_q == 0) return ok();
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, causal, sinks, num_q_heads)) != SA_OK) return s;
    hipError_t e;
    const sa::StateSlots ss{kv_chunk_size, max_num_chunks, max_num_chunks, 0, 1};
    if (mfma)
        e = sa::launch_mfma_prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, batch,
                                          num_q_heads, num_kv_heads, max_seqlen_q, max_seqlen_k, ss,
                                          sm_scale, causal, part_m, part_d, part_acc, st);
    else
        e = sa::launch_generic_prefill_split(dtype == SA_BF16, q, k, v, sinks, cu_seqlens_q,
                                             cu_seqlens_k, batch, num_q_heads, num_kv_heads,
                                             max_seqlen_q, ss, sm_scale, causal, part_m, part_d,
                                             part_acc, st);
    return finish_launch(e, st, "sink_attn_prefill_split");
}

sa_status_t sink_attn_prefill_state(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k, float sm_scale,
                                    int32_t causal, int32_t include_sink, int32_t slot,
                                    int32_t num_slots, float* part_m, float* part_d,
                                    float* part_acc, void* stream) {
    sa_status_t s;
    if ((s = check_dtype(dtype)) != SA_OK) return s;
    if (!q || !k || !v || !sinks || !cu_seqlens_q || !cu_seqlens_k || !part_m || !part_d ||
        !part_acc)
        return fail(SA_EINVAL, "sink_attn_prefill_state: null pointer argument");
    if ((s = check_alignment("sink_attn_prefill_state", q, k, v, part_acc, nullptr, 1)) != SA_OK)
        return s;
    if ((s = check_heads(batch, num_q_heads, num_kv_heads, head_dim)) != SA_OK) return s;
    if (max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(SA_EINVAL, "max_seqlen_q/max_seqlen_k must be >= 0");
    if (causal != 0 && causal != 1) return fail(SA_EINVAL, "causal must be 0 or 1");
    if (include_sink != 0 && include_sink != 1) return fail(SA_EINVAL, "include_sink must be 0 or 1");
    if (num_slots < 1) return fail(SA_EINVAL, "num_slots must be >= 1, got %d", num_slots);
    if (slot < 0 || slot >= num_slots)
        return fail(SA_EINVAL, "slot %d is outside [0, num_slots = %d)", slot, num_slots);
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SA_EINVAL, "sm_scale must be finite and > 0");
    const int group = num_q_heads / num_kv_heads;
    const bool mfma = dtype == SA_BF16 && sa::mfma_prefill_supported(group);
    if (mfma) {
        if ((s = check_grid((int64_t)batch * num_kv_heads * qblocks_bound(max_seqlen_q), 64 * group,
                            "sink_attn_prefill_state")) != SA_OK)
            return s;
    } else if ((s = check_grid(max_seqlen_q, 64, "sink_attn_prefill_state")) != SA_OK) {
        return s;
    }
    if (max_seqlen_q == 0) return ok();
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, causal, sinks, num_q_heads)) != SA_OK) return s;
    // one chunk starting at key 0 that no sequence outgrows
    const sa::StateSlots ss{0x7fffffff, 1, num_slots, slot, include_sink};
    hipError_t e;
    if (mfma)
        e = sa::launch_mfma_prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, batch,
                                          num_q_heads, num_kv_heads, max_seqlen_q, max_seqlen_k, ss,
                                          sm_scale, causal, part_m, part_d, part_acc, st);
    else
        e = sa::launch_generic_prefill_split(dtype == SA_BF16, q, k, v, sinks, cu_seqlens_q,
                                             cu_seqlens_k, batch, num_q_heads, num_kv_heads,
                                             max_seqlen_q, ss, sm_scale, causal, part_m, part_d,
                                             part_acc, st);
    return finish_launch(e, st, "sink_attn_prefill_state");
}

sa_status_t sink_attn_merge_rows(sa_dtype_t out_dtype, const float* part_m, const float* part_d,
                                 const float* part_acc, int32_t num_rows, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_num_chunks, void* out, float* lse,
                                 void* stream) {
    sa_status_t s;
    if ((s = check_dtype(out_dtype)) != SA_OK) return s;
    if (!part_m || !part_d || !part_acc || !out)
        return fail(SA_EINVAL, "sink_attn_merge_rows: null pointer argument");
    if (num_rows < 0) return fail(SA_EINVAL, "num_rows must be >= 0, got %d", num_rows);
    if (num_q_heads < 1) return fail(SA_EINVAL, "num_q_heads must be >= 1");
    if (head_dim != 64) return fail(SA_EUNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
    if (max_num_chunks < 1) return fail(SA_EINVAL, "max_num_chunks must be >= 1");
    if ((s = check_grid(((int64_t)num_rows * num_q_heads + 3) / 4, 256, "sink_attn_merge_rows")) != SA_OK)
        return s;
    if (num_rows == 0) return ok();
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_merge(out_dtype == SA_BF16, part_m, part_d, part_acc, nullptr, 1,
                                    max_num_chunks, num_rows, num_q_heads, out, lse, st);
    return finish_launch(e, st, "sink_attn_merge_rows");
}

}  // extern "C"

namespace {

// kv_chunk_size == 0 (proportional blocks) is valid only where allow_balanced is set.
sa_status_t check_split_args(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                             const float* sinks, const int32_t* cu_seqlens_k, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_seqlen_k, int32_t kv_chunk_size, int32_t max_num_chunks,
                             float sm_scale, const float* part_m, const float* part_d,
                             const float* part_acc, bool allow_balanced) {
    sa_status_t s;
    if ((s = check_dtype(dtype)) != SA_OK) return s;
    if (!q || !k || !v || !sinks || !cu_seqlens_k || !part_m || !part_d || !part_acc)
        return fail(SA_EINVAL, "decode: null pointer argument");
    if ((s = check_alignment("decode", q, k, v, part_acc, nullptr, 1)) != SA_OK) return s;
    if ((s = check_heads(batch, num_q_heads, num_kv_heads, head_dim)) != SA_OK) return s;
    if (kv_chunk_size < 0 || (kv_chunk_size == 0 && !allow_balanced))
        return fail(SA_EINVAL, "kv_chunk_size must be >= %d, got %d", allow_balanced ? 0 : 1, kv_chunk_size);
    if (max_seqlen_k < 0) return fail(SA_EINVAL, "max_seqlen_k must be >= 0");
    if (kv_chunk_size > 0) {
        const int64_t need = max_seqlen_k == 0 ? 1 : ((int64_t)max_seqlen_k + kv_chunk_size - 1) / kv_chunk_size;
        if (max_num_chunks < need)
            return fail(SA_EINVAL, "max_num_chunks (%d) < ceil(max_seqlen_k / kv_chunk_size) = %lld",
                        max_num_chunks, (long long)need);
        if ((s = check_chunk_span(kv_chunk_size, max_num_chunks, "decode")) != SA_OK) return s;
    } else if (max_num_chunks < 1) {
        return fail(SA_EINVAL, "max_num_chunks must be >= 1, got %d", max_num_chunks);
    }
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SA_EINVAL, "sm_scale must be finite and > 0");
    // fixed chunks: one workgroup per (sequence, chunk slot, block of eight waves, one
    // wave per KV head or slice of at most 16 query heads)
    if (kv_chunk_size > 0 &&
        (s = check_grid((int64_t)batch * max_num_chunks * ((num_q_heads + 7) / 8), 512, "decode")) != SA_OK)
        return s;
    return SA_OK;
}

// Compute units of the current device (the balanced decode gives each one range).
int compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev].load(std::memory_order_relaxed) > 0)
        return cached[dev].load(std::memory_order_relaxed);
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The key blocks of a one-call decode.  kv_chunk_size > 0: those chunks.  0:
// proportional blocks (matrix-core path, two or more state slots per sequence),
// one workgroup per compute unit (all of them streaming at once, none holding two
// while another idles): the ranges are whole rounds of one workgroup per compute
// unit, one round when the batch is at most half of one, else enough rounds that
// at least half a round is left to share out by key count; elsewhere the smallest
// fixed chunk the slots allow.
sa_status_t decode_plan(sa_dtype_t dtype, int32_t batch, int32_t hq, int32_t hkv,
                        int32_t max_seqlen_k, int32_t kv_chunk_size, int32_t max_num_chunks,
                        sa::DecodePlan* plan) {
    if (kv_chunk_size > 0) {
        *plan = sa::DecodePlan{kv_chunk_size, 0, max_seqlen_k, max_num_chunks};
        return SA_OK;
    }
    if (dtype == SA_BF16 && sa::mfma_decode_supported(hq / hkv) && max_num_chunks >= 2) {
        const int head_blocks = sa::mfma_decode_head_blocks(hq, hkv);
        const int per_round = std::max(1, compute_units() / head_blocks);
        const int64_t ranges = (int64_t)per_round * ((batch + per_round / 2 + per_round - 1) / per_round);
        sa_status_t s = check_grid(ranges * head_blocks, 512, "sink_attn_decode");
        if (s != SA_OK) return s;
        *plan = sa::DecodePlan{0, (int)ranges, max_seqlen_k, max_num_chunks};
        return SA_OK;
    }
    const int32_t chunk = std::max<int32_t>(1, max_seqlen_k / max_num_chunks + (max_seqlen_k % max_num_chunks != 0));
    sa_status_t s = check_chunk_span(chunk, max_num_chunks, "sink_attn_decode");
    if (s != SA_OK) return s;
    if (dtype == SA_BF16 && sa::mfma_decode_supported(hq / hkv) &&
        (s = check_grid((int64_t)batch * max_num_chunks * ((hq + 7) / 8), 512, "sink_attn_decode")) != SA_OK)
        return s;
    *plan = sa::DecodePlan{chunk, 0, max_seqlen_k, max_num_chunks};
    return SA_OK;
}

hipError_t launch_split(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                        const float* sinks, const int32_t* cu_seqlens_k, int32_t batch,
                        int32_t hq, int32_t hkv, const sa::DecodePlan& plan, float sm_scale,
                        float* part_m, float* part_d, float* part_acc, hipStream_t st) {
    if (dtype == SA_BF16 && sa::mfma_decode_supported(hq / hkv))
        return sa::launch_mfma_decode_plan(q, k, v, sinks, cu_seqlens_k, batch, hq, hkv, plan,
                                           sm_scale, part_m, part_d, part_acc, st);
    // the vector-ALU path takes fixed chunks only (decode_plan never gives it ranges)
    return sa::launch_generic_decode_split(dtype == SA_BF16, q, k, v, sinks, cu_seqlens_k, batch,
                                           hq, hkv, plan.chunk, plan.max_chunks, sm_scale, part_m,
                                           part_d, part_acc, st);
}

}  // namespace

extern "C" {

sa_status_t sink_attn_decode_split(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                                   const float* sinks, const int32_t* cu_seqlens_k, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_seqlen_k, int32_t kv_chunk_size,
                                   int32_t max_num_chunks, float sm_scale, float* part_m,
                                   float* part_d, float* part_acc, void* stream) {
    sa_status_t s = check_split_args(dtype, q, k, v, sinks, cu_seqlens_k, batch, num_q_heads,
                                     num_kv_heads, head_dim, max_seqlen_k, kv_chunk_size,
                                     max_num_chunks, sm_scale, part_m, part_d, part_acc, false);
    if (s != SA_OK) return s;
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, nullptr, cu_seqlens_k, batch, 1, max_seqlen_k, 0, sinks, num_q_heads)) != SA_OK) return s;
    const sa::DecodePlan plan{kv_chunk_size, 0, max_seqlen_k, max_num_chunks};
    hipError_t e = launch_split(dtype, q, k, v, sinks, cu_seqlens_k, batch, num_q_heads,
                                num_kv_heads, plan, sm_scale, part_m, part_d, part_acc, st);
    return finish_launch(e, st, "sink_attn_decode_split");
}

sa_status_t sink_attn_decode(sa_dtype_t dtype, const void* q, const void* k, const void* v,
                             const float* sinks, const int32_t* cu_seqlens_k, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_seqlen_k, int32_t kv_chunk_size, int32_t max_num_chunks,
                             float sm_scale, float* part_m, float* part_d, float* part_acc,
                             void* out, float* lse, void* stream) {
    sa_status_t s = check_split_args(dtype, q, k, v, sinks, cu_seqlens_k, batch, num_q_heads,
                                     num_kv_heads, head_dim, max_seqlen_k, kv_chunk_size,
                                     max_num_chunks, sm_scale, part_m, part_d, part_acc, true);
    if (s != SA_OK) return s;
    if (!out) return fail(SA_EINVAL, "sink_attn_decode: null pointer argument");
    if ((s = check_device()) != SA_OK) return s;
    sa::DecodePlan plan;
    if ((s = decode_plan(dtype, batch, num_q_heads, num_kv_heads, max_seqlen_k, kv_chunk_size,
                         max_num_chunks, &plan)) != SA_OK)
        return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, nullptr, cu_seqlens_k, batch, 1, max_seqlen_k, 0, sinks, num_q_heads)) != SA_OK) return s;
    hipError_t e = launch_split(dtype, q, k, v, sinks, cu_seqlens_k, batch, num_q_heads,
                                num_kv_heads, plan, sm_scale, part_m, part_d, part_acc, st);
    if (e == hipSuccess)
        e = sa::launch_merge_plan(dtype == SA_BF16, part_m, part_d, part_acc, cu_seqlens_k, plan,
                                  batch, num_q_heads, out, lse, st);
    return finish_launch(e, st, "sink_attn_decode");
}

sa_status_t sink_attn_decode_noalloc(sa_dtype_t dtype, const void* q, const void* k,
                                     const void* v, const float* sinks,
                                     const int32_t* cu_seqlens_k, int32_t batch,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t max_seqlen_k, float sm_scale, void* out, float* lse,
                                     void* stream) {
    sa_status_t s;
    if ((s = check_dtype(dtype)) != SA_OK) return s;
    if (!q || !k || !v || !sinks || !cu_seqlens_k || !out)
        return fail(SA_EINVAL, "sink_attn_decode_noalloc: null pointer argument");
    if ((s = check_alignment("sink_attn_decode_noalloc", q, k, v, nullptr, nullptr, 1)) != SA_OK)
        return s;
    if ((s = check_heads(batch, num_q_heads, num_kv_heads, head_dim)) != SA_OK) return s;
    if (max_seqlen_k < 0) return fail(SA_EINVAL, "max_seqlen_k must be >= 0");
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(SA_EINVAL, "sm_scale must be finite and > 0");
    // State slots per (sequence, head) in the fixed array: acc [pairs * slots * D] floats,
    // then m and d, each padded to 256 bytes.
    const int64_t pairs = (int64_t)batch * num_q_heads;
    const int64_t floats = (int64_t)(sa::kDecodeScratchBytes / sizeof(float));
    const int64_t fit = (floats - 128) / (pairs * (head_dim + 2));
    if (fit < 1)
        return fail(SA_EINVAL,
                    "sink_attn_decode_noalloc: batch * num_q_heads = %lld needs more than the "
                    "%zu-byte state array (at most %lld)", (long long)pairs,
                    sa::kDecodeScratchBytes, (long long)((floats - 128) / (head_dim + 2)));
    if ((s = check_device()) != SA_OK) return s;
    // as many slots as one sequence can be given (blocks beyond one per sequence, plus two)
    const int units = compute_units();
    const int64_t ranges = (int64_t)units * ((batch + units / 2 + units - 1) / units);
    const int32_t slots = (int32_t)std::max<int64_t>(1, std::min(ranges - batch + 2, fit));
    sa::DecodePlan plan;
    if ((s = decode_plan(dtype, batch, num_q_heads, num_kv_heads, max_seqlen_k, 0, slots,
                         &plan)) != SA_OK)
        return s;
    float* base = nullptr;
    hipError_t e = sa::decode_scratch(&base);
    if (e != hipSuccess)
        return fail(SA_ELAUNCH, "sink_attn_decode_noalloc: state array: %s", hipGetErrorString(e));
    const int64_t states = pairs * slots;
    float* part_acc = base;
    float* part_m = part_acc + states * head_dim;
    float* part_d = part_m + (states + 63) / 64 * 64;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = debug_check_inputs(st, nullptr, cu_seqlens_k, batch, 1, max_seqlen_k, 0, sinks, num_q_heads)) != SA_OK) return s;
    e = launch_split(dtype, q, k, v, sinks, cu_seqlens_k, batch, num_q_heads, num_kv_heads, plan,
                     sm_scale, part_m, part_d, part_acc, st);
    if (e == hipSuccess)
        e = sa::launch_merge_plan(dtype == SA_BF16, part_m, part_d, part_acc, cu_seqlens_k, plan,
                                  batch, num_q_heads, out, lse, st);
    return finish_launch(e, st, "sink_attn_decode_noalloc");
}

sa_status_t sink_attn_merge(sa_dtype_t out_dtype, const float* part_m, const float* part_d,
                            const float* part_acc, const int32_t* cu_seqlens_k,
                            int32_t kv_chunk_size, int32_t max_num_chunks, int32_t batch,
                            int32_t num_q_heads, int32_t head_dim, void* out, float* lse,
                            void* stream) {
    sa_status_t s;
    if ((s = check_dtype(out_dtype)) != SA_OK) return s;
    if (!part_m || !part_d || !part_acc || !cu_seqlens_k || !out)
        return fail(SA_EINVAL, "sink_attn_merge: null pointer argument");
    if (batch < 1 || batch > 65535) return fail(SA_EINVAL, "batch must be in [1, 65535], got %d", batch);
    if (num_q_heads < 1) return fail(SA_EINVAL, "num_q_heads must be >= 1");
    if ((s = check_grid(((int64_t)batch * num_q_heads + 3) / 4, 256, "sink_attn_merge")) != SA_OK)
        return s;
    if (head_dim != 64) return fail(SA_EUNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
    if (kv_chunk_size < 1) return fail(SA_EINVAL, "kv_chunk_size must be >= 1, got %d", kv_chunk_size);
    if (max_num_chunks < 1) return fail(SA_EINVAL, "max_num_chunks must be >= 1");
    if ((s = check_chunk_span(kv_chunk_size, max_num_chunks, "sink_attn_merge")) != SA_OK) return s;
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_merge(out_dtype == SA_BF16, part_m, part_d, part_acc, cu_seqlens_k,
                                    kv_chunk_size, max_num_chunks, batch, num_q_heads, out, lse, st);
    return finish_launch(e, st, "sink_attn_merge");
}

sa_status_t moe_topk_softmax(const void* logits, int64_t num_tokens, int32_t num_experts,
                             int32_t k, int32_t* indices, void* weights, void* stream) {
    if (num_tokens < 0) return fail(SA_EINVAL, "num_tokens must be >= 0");
    if (!sa::topk_softmax_supported(num_experts))
        return fail(SA_EUNSUPPORTED, "num_experts %d is not supported (8, 16, ..., 512)", num_experts);
    if (k < 1 || k > 8 || k > num_experts)
        return fail(SA_EINVAL, "k must be in [1, min(8, num_experts)], got %d", k);
    if (num_tokens == 0) return ok();  // nothing to read or write: pointers may be null
    if (!logits || !indices || !weights) return fail(SA_EINVAL, "moe_topk_softmax: null pointer argument");
    if (reinterpret_cast<uintptr_t>(logits) % 16 != 0)
        return fail(SA_EINVAL, "moe_topk_softmax: logits must be 16-byte aligned");
    sa_status_t s;
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_topk_softmax(logits, num_tokens, num_experts, k, indices, weights, st);
    return finish_launch(e, st, "moe_topk_softmax");
}

sa_status_t qkv_bias_rope(const void* qkv, const void* bias, const int32_t* positions,
                          const float* cos_sin, int64_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t table_rows, void* q,
                          void* k, void* v, void* stream) {
    if (num_tokens < 0) return fail(SA_EINVAL, "num_tokens must be >= 0");
    if (num_q_heads < 1 || num_kv_heads < 1) return fail(SA_EINVAL, "head counts must be >= 1");
    if (head_dim != 64) return fail(SA_EUNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
    if (table_rows < 1) return fail(SA_EINVAL, "table_rows must be >= 1");
    const int64_t heads = (int64_t)num_q_heads + 2 * (int64_t)num_kv_heads;
    sa_status_t s;
    // eight 16-byte pieces per head, two per thread: num_tokens * heads * 4 work-items
    // (rounded up to whole blocks of 256), below 2^32
    if (num_tokens > ((int64_t)0xFFFFFFFFLL - 512) / (heads * 4))
        return fail(SA_EINVAL, "qkv_bias_rope: num_tokens * heads * 4 exceeds the 2^32 work-item grid limit");
    if (num_tokens == 0) return ok();  // nothing to read or write: pointers may be null
    if (!qkv || !bias || !positions || !cos_sin || !q || !k || !v)
        return fail(SA_EINVAL, "qkv_bias_rope: null pointer argument");
    for (const void* p : {qkv, bias, (const void*)cos_sin, (const void*)q, (const void*)k, (const void*)v})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(SA_EINVAL, "qkv_bias_rope: qkv, bias, cos_sin, q, k and v must be 16-byte aligned");
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_qkv_rope(qkv, bias, positions, cos_sin, num_tokens, num_q_heads,
                                       num_kv_heads, table_rows, q, k, v, st);
    return finish_launch(e, st, "qkv_bias_rope");
}

sa_status_t sink_attn_read_probe(const void* buf, int64_t bytes, int32_t num_blocks,
                                 uint32_t* out, void* stream) {
    if ((!buf && bytes != 0) || !out)
        return fail(SA_EINVAL, "sink_attn_read_probe: null pointer argument");
    if (bytes < 0 || bytes % 16 != 0)
        return fail(SA_EINVAL, "sink_attn_read_probe: bytes must be >= 0 and a multiple of 16");
    if (num_blocks < 1 || num_blocks > 65535)
        return fail(SA_EINVAL, "sink_attn_read_probe: num_blocks must be in [1, 65535]");
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return fail(SA_EINVAL, "sink_attn_read_probe: buf must be 16-byte aligned");
    sa_status_t s;
    if ((s = check_device()) != SA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_read_probe(buf, bytes, num_blocks, out, st);
    return finish_launch(e, st, "sink_attn_read_probe");
}

}  // extern "C"
