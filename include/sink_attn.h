/*
 * sink_attn.h -- C ABI of the MI355X (gfx950) library for grouped-query
 * attention with a learned per-head attention sink.
 *
 * The operation is the one described in "GPT-OSS on day 0" (Perplexity),
 * section "Kernels for GPT-OSS / Sink attention":
 *
 *     attn = softmax(q k^T * sm_scale + sink) V
 *
 * where each query head h owns one pre-trained sink logit (section
 * "Attention and MLP architecture": GQA with attention sinks; each head
 * carries a sink parameter that enters its softmax).  The library reads the
 * sink as one more softmax entry with a zero value vector: it is added to
 * the denominator, it is NOT multiplied by sm_scale and it is in natural-log
 * units.  That is what starting the online softmax's running maximum at the
 * head's sink value (with the running scale at 1) computes, as the same
 * section describes; when the keys are split into blocks along the sequence
 * the sink enters the first block only.
 *
 * Grouped-query attention: with Hq query heads and Hkv key/value heads,
 * query head h reads key/value head h / (Hq / Hkv).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer; arrays are contiguous and
 *     row-major.  Token-major packed layout: q [total_q, Hq, D],
 *     k and v [total_k, Hkv, D].  head_dim D = 64 is supported.
 *   - cu_seqlens_* are device int32 arrays of batch+1 nondecreasing
 *     absolute row offsets: sequence b owns rows [cu[b], cu[b+1]).
 *   - The caller allocates and owns every buffer (including the split-KV
 *     partial buffers).  The library never allocates, frees or synchronises.
 *     Inputs are read-only; outputs must not alias inputs.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the default stream).
 *   - Host-checkable errors are reported before anything is launched:
 *     SA_EINVAL for invalid arguments, SA_EUNSUPPORTED for a valid but
 *     unimplemented combination (dtype, head_dim, group size), SA_ELAUNCH if
 *     the HIP runtime rejects the launch or no device is present.  The text
 *     of the last error of the calling thread is returned by
 *     sink_attn_last_error().
 *   - sm_scale must be finite and > 0 (SA_EINVAL otherwise).
 *   - Alignment: q, k, v and part_acc must be 16-byte aligned, and the out of
 *     sink_attn_prefill 8-byte aligned (the kernels move them in pieces of that
 *     size); SA_EINVAL otherwise.  Allocations from hipMalloc (or torch) and
 *     row-offset views of them meet this.
 *   - Device-resident preconditions cannot be checked without a
 *     synchronisation and are the caller's duty: monotone cu_seqlens,
 *     L_q <= L_k for every sequence under causal masking, per-sequence
 *     lengths no larger than the max_seqlen_* bounds given, sinks that are
 *     finite or -inf (never +inf or NaN).  Broken ones give wrong results, not
 *     out-of-bounds accesses: no kernel reads or writes outside the rows and
 *     slots the host-side arguments describe.
 *   - Debugging aid: with SINK_ATTN_DEBUG=1 in the environment (read once per
 *     process), the attention entry points synchronise `stream`, copy the
 *     sequence offsets and sinks to the host and check the preconditions
 *     above (SA_EINVAL), and synchronise again after the launch so that a
 *     failing kernel is reported as SA_ELAUNCH.  This is slow and must not be
 *     used while the stream is being captured into a graph.
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SA_OK = 0,
    SA_EINVAL = 1,
    SA_EUNSUPPORTED = 2,
    SA_ELAUNCH = 3
} sa_status_t;

typedef enum {
    SA_FP32 = 0,   /* IEEE float32 */
    SA_BF16 = 1    /* bfloat16 (upper 16 bits of a float32), round-to-nearest-even on output */
} sa_dtype_t;

/*
 * Attention with sinks over a packed varlen batch (prefill, or any mix of
 * prefill chunks and single-token decodes).
 *
 * The section's operation for every query row: with L_q queries and L_k keys
 * in sequence b, row i (0-based within the sequence) sees keys
 * 0 .. L_k - L_q + i when `causal` is nonzero (bottom-right alignment: the
 * row sits at key position L_k - L_q + i), and all L_k keys otherwise.
 *
 *   q      [total_q, Hq, D]   dtype
 *   k, v   [total_k, Hkv, D]  dtype
 *   sinks  [Hq] float32, natural-log units, finite or -inf
 *   cu_seqlens_q, cu_seqlens_k  [batch+1] int32
 *   max_seqlen_q, max_seqlen_k  host-side upper bounds of L_q and L_k (grid sizing)
 *   out    [total_q, Hq, D]   dtype; rows with no visible key and sink = -inf get 0
 *   lse    nullable; [total_q, Hq] float32: ln(e^sink + sum_j e^(s_j)), -inf if empty
 */
sa_status_t sink_attn_prefill(sa_dtype_t dtype, const void *q, const void *k, const void *v,
                              const float *sinks, const int32_t *cu_seqlens_q,
                              const int32_t *cu_seqlens_k, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, float sm_scale, int32_t causal, void *out,
                              float *lse, void *stream);

/*
 * Split-KV decode, first pass: one query token per sequence, the keys of each
 * sequence cut into blocks ("chunks") along the sequence, as the section
 * describes for attention parallelised along the KV length.  Chunk c of
 * sequence b covers keys [c*C, min((c+1)*C, L_b)) with C = kv_chunk_size;
 * nchunks(b) = max(1, ceil(L_b / C)) (chunk 0 always exists because it
 * carries the sink).  The running maximum of chunk 0 starts at the head's
 * sink, that of every other chunk at -inf; the running scale starts at 1.
 *
 *   q          [batch, Hq, D] dtype
 *   k, v       [total_k, Hkv, D] dtype, sequence b's keys at rows [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *   max_seqlen_k  host-side upper bound of L_b
 *   max_num_chunks  slots per (b, h) in the partial buffers; must be >= ceil(max_seqlen_k / C),
 *                   and max_num_chunks * C must stay below 2^31 (SA_EINVAL otherwise)
 *   part_m, part_d  [batch, Hq, max_num_chunks] float32
 *   part_acc        [batch, Hq, max_num_chunks, D] float32
 * For every c < nchunks(b) the call writes the state after chunk c's keys:
 * m (natural-log units), d = sum over the chunk of e^(s_j - m) (plus
 * e^(sink - m) in chunk 0) and acc = sum of e^(s_j - m) v_j (unnormalised).
 * A chunk whose state holds no mass has m = -inf.  Slots c >= nchunks(b) are
 * not written.
 */
sa_status_t sink_attn_decode_split(sa_dtype_t dtype, const void *q, const void *k, const void *v,
                                   const float *sinks, const int32_t *cu_seqlens_k, int32_t batch,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_seqlen_k, int32_t kv_chunk_size,
                                   int32_t max_num_chunks, float sm_scale, float *part_m,
                                   float *part_d, float *part_acc, void *stream);

/*
 * Split-KV decode, second pass: the log-sum-exp combination of the chunk
 * states written by sink_attn_decode_split (same cu_seqlens_k, chunk size and
 * max_num_chunks):  M = max_c m_c,  w_c = e^(m_c - M),
 * out = sum_c w_c acc_c / sum_c w_c d_c,  lse = M + ln sum_c w_c d_c;
 * out = 0 and lse = -inf when every chunk is at -inf.
 *
 *   out  [batch, Hq, D] out_dtype
 *   lse  nullable; [batch, Hq] float32
 */
sa_status_t sink_attn_merge(sa_dtype_t out_dtype, const float *part_m, const float *part_d,
                            const float *part_acc, const int32_t *cu_seqlens_k,
                            int32_t kv_chunk_size, int32_t max_num_chunks, int32_t batch,
                            int32_t num_q_heads, int32_t head_dim, void *out, float *lse,
                            void *stream);

/*
 * Split-KV decode in one call: a split pass then the log-sum-exp merge, enqueued
 * back to back on `stream`.  The section splits each sequence's keys into blocks
 * along the KV length, the sink entering the first block only; the result does not
 * depend on where the blocks fall.
 *
 *   kv_chunk_size > 0  fixed chunks: exactly sink_attn_decode_split followed by
 *             sink_attn_merge (same arguments, same partial states, same result),
 *             and the same bounds on max_num_chunks.
 *   kv_chunk_size == 0 proportional blocks, chosen by the library so that one
 *             launch gives every compute unit about the same number of key bytes:
 *             each sequence gets at least one block and the remaining blocks of the
 *             launch in proportion to its key count, and splits its keys evenly
 *             over them (contiguous blocks, the first one holding key 0 and the
 *             sink).  At most max_num_chunks (>= 1) blocks per sequence; more slots
 *             allow a finer balance (a sequence can be given up to the compute-unit
 *             count plus one blocks; with max_num_chunks = 1 every sequence is one
 *             block).  bf16 inputs only; for float32 inputs this picks the smallest
 *             fixed chunk the slots allow.
 *   part_m, part_d, part_acc  caller-owned workspace of max_num_chunks state slots
 *             per (sequence, head): [batch, Hq, max_num_chunks] and
 *             [batch, Hq, max_num_chunks, D] float32 in size.  With fixed chunks
 *             they hold the chunk states after the call, laid out as for
 *             sink_attn_decode_split; with proportional blocks their content and
 *             layout are the library's own.
 *   out       [batch, Hq, D] dtype;  lse nullable [batch, Hq] float32.
 * Errors: those of sink_attn_decode_split (kv_chunk_size >= 0 here), and SA_EINVAL
 * for a null `out` or max_num_chunks < 1.
 */
sa_status_t sink_attn_decode(sa_dtype_t dtype, const void *q, const void *k, const void *v,
                             const float *sinks, const int32_t *cu_seqlens_k, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_seqlen_k, int32_t kv_chunk_size, int32_t max_num_chunks,
                             float sm_scale, float *part_m, float *part_d, float *part_acc,
                             void *out, float *lse, void *stream);

/*
 * For callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): sink_attn_decode with
 * kv_chunk_size = 0 (proportional blocks), its block states kept in a fixed device
 * array of SA_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, instead of a caller workspace.  The call itself allocates
 * nothing: no hipMalloc, no hipFree.
 *
 *   Arguments and result as for sink_attn_decode; the library chooses the state
 *   slots per sequence (as many as fit in the array, up to the most one sequence
 *   can be given).
 * Limit: batch * num_q_heads * (head_dim + 2) * 4 bytes (one slot per sequence and
 * head) must fit in the array: at most 508,398 (sequence, head) pairs at head_dim
 * 64; beyond it SA_EINVAL, before anything is launched.
 * Every call on one GPU shares that GPU's array and leaves its states there; no
 * call needs it cleared.  Calls that overlap on one GPU (on different streams, or
 * from several host threads) race on it: order them on one stream.  The first call
 * on a device looks up the array's address on that device.
 */
#define SA_DECODE_SCRATCH_BYTES (128u << 20)
sa_status_t sink_attn_decode_noalloc(sa_dtype_t dtype, const void *q, const void *k,
                                     const void *v, const float *sinks,
                                     const int32_t *cu_seqlens_k, int32_t batch,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t max_seqlen_k, float sm_scale, void *out, float *lse,
                                     void *stream);

/*
 * Split-KV prefill, first pass: the prefill problem of sink_attn_prefill with the
 * keys of every sequence cut into chunks of kv_chunk_size keys, chunk c covering
 * keys [c*C, min((c+1)*C, L_k)) -- the split along the KV length of "GPT-OSS on
 * day 0" (Perplexity), Kernels for GPT-OSS / Sink attention, with the sink in the
 * first block only.  For every query row r (absolute row in q), query head h and
 * chunk c < max_num_chunks it writes the state (m, d, acc) after the keys of
 * chunk c that row r may see (the whole chunk, or its causal part); the sink is
 * part of chunk 0's state only.  A chunk the row cannot see (and every slot
 * c >= ceil(L_k / C)) holds the empty state m = -inf, d = 0, acc = 0, except
 * that chunk 0 always carries the sink (m = sink, d = 1, acc = 0 when no key is
 * visible).  m is in natural-log units, acc is unnormalised.
 *
 *   Arguments as for sink_attn_prefill, plus kv_chunk_size >= 1 and
 *   max_num_chunks >= ceil(max_seqlen_k / kv_chunk_size) (>= 1), with
 *   max_num_chunks * kv_chunk_size below 2^31.
 *   part_m, part_d  [total_q, Hq, max_num_chunks] float32 (caller-owned)
 *   part_acc        [total_q, Hq, max_num_chunks, D] float32 (caller-owned)
 * Errors as for sink_attn_prefill; SA_EINVAL for a too small max_num_chunks or a
 * launch grid beyond the device limits.
 */
sa_status_t sink_attn_prefill_split(sa_dtype_t dtype, const void *q, const void *k, const void *v,
                                    const float *sinks, const int32_t *cu_seqlens_q,
                                    const int32_t *cu_seqlens_k, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t kv_chunk_size, int32_t max_num_chunks, float sm_scale,
                                    int32_t causal, float *part_m, float *part_d, float *part_acc,
                                    void *stream);

/*
 * State of each query row's attention over the keys one call sees, written to one
 * slot of a caller-chosen slot buffer, for cascade attention: the new tokens of
 * many sequences attend a shared cached prefix in one call (all queries packed as
 * one sequence over the prefix keys, non-causal) and their own keys in another
 * (per sequence, causal), each call writing its own slot; sink_attn_merge_rows
 * then combines the slots.  This is the section's split along the KV sequence
 * with the two key sets as the blocks; the sink belongs to exactly one of them,
 * so it enters this call's states only when include_sink is 1.
 *
 * Keys, masking and arguments are those of sink_attn_prefill (one block holding
 * every visible key).  For every row r and head h the state after all of the
 * row's visible keys, (m natural-log units, d, unnormalised acc), goes to slot
 * `slot` of
 *   part_m, part_d  [total_q, Hq, num_slots] float32;  part_acc [total_q, Hq, num_slots, D]
 * and no other slot is written.  A row with no visible key and no sink gets
 * (m = -inf, d = 0, acc = 0).
 * Errors: those of sink_attn_prefill, plus SA_EINVAL for null partial buffers,
 * num_slots < 1, slot outside [0, num_slots), include_sink not 0 or 1.
 * max_seqlen_q = 0 does nothing.
 */
sa_status_t sink_attn_prefill_state(sa_dtype_t dtype, const void *q, const void *k, const void *v,
                                    const float *sinks, const int32_t *cu_seqlens_q,
                                    const int32_t *cu_seqlens_k, int32_t batch,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k, float sm_scale,
                                    int32_t causal, int32_t include_sink, int32_t slot,
                                    int32_t num_slots, float *part_m, float *part_d,
                                    float *part_acc, void *stream);

/*
 * Log-sum-exp combination of every slot of per-row chunk states, as written by
 * sink_attn_prefill_split or sink_attn_prefill_state (the same combination as sink_attn_merge: with
 * M = max_c m_c, out = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) d_c and
 * lse = M + ln sum_c e^(m_c - M) d_c; all m_c = -inf gives out = 0, lse = -inf).
 *
 *   part_m, part_d  [num_rows, Hq, max_num_chunks] float32;  part_acc [.., D]
 *   out             [num_rows, Hq, D] out_dtype;  lse nullable [num_rows, Hq] float32
 * Errors: SA_EINVAL for null pointers, num_rows < 0, Hq < 1, max_num_chunks < 1;
 * SA_EUNSUPPORTED for head_dim != 64.  num_rows = 0 does nothing.
 */
sa_status_t sink_attn_merge_rows(sa_dtype_t out_dtype, const float *part_m, const float *part_d,
                                 const float *part_acc, int32_t num_rows, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_num_chunks, void *out, float *lse,
                                 void *stream);

/* Text of the calling thread's last non-OK status ("" if none).  Valid until the next call. */
const char *sink_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
