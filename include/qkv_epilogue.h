/*
 * qkv_epilogue.h -- C ABI of the pre-attention epilogue, in the same library as
 * sink_attn.h (libsinkattn.so, gfx950).
 *
 * "GPT-OSS on day 0" (Perplexity), architecture list: the QKV projections have
 * biases and positions are encoded with YaRN rotary embeddings.  This call takes
 * the fused QKV projection output, adds the bias and applies the rotary
 * embedding to the query and key heads, writing q, k and v in the layouts
 * sink_attn_prefill / sink_attn_decode read.  The YaRN frequencies and attention
 * scale are folded into the caller's table; the pages give no YaRN constants.
 */
#ifndef QKV_EPILOGUE_H
#define QKV_EPILOGUE_H

#include <stdint.h>

#include "sink_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * qkv        [num_tokens, (Hq + 2 Hkv) * D] bf16 (device): per token the Hq query
 *            heads, then the Hkv key heads, then the Hkv value heads, D = 64 each
 * bias       [(Hq + 2 Hkv) * D] bf16 (device)
 * positions  [num_tokens] int32 (device): each token's position; values outside
 *            [0, table_rows) take the nearest row
 * cos_sin    [table_rows, D] float32 (device): row p = cos(p w_i) for i < D/2, then
 *            sin(p w_i) (frequencies and scale as the caller's YaRN setup gives them)
 * q [num_tokens, Hq, D], k [num_tokens, Hkv, D], v [num_tokens, Hkv, D] bf16 (device, written)
 * With x = qkv + bias in float32: query and key heads become
 *   y_i = x_i c_i - x_{i+D/2} s_i,  y_{i+D/2} = x_{i+D/2} c_i + x_i s_i  (i < D/2),
 * value heads y = x; results are rounded to bf16 (round to nearest even).
 * qkv, bias, cos_sin, q, k and v must be 16-byte aligned (rows are read and written
 * as 16-byte vectors); the caller keeps ownership of every buffer.  The call is
 * enqueued on `stream` (NULL: the default stream) and returns before it runs.
 * Errors: SA_EINVAL for null or misaligned pointers (num_tokens > 0), num_tokens < 0, head counts
 * < 1, table_rows < 1 or a grid beyond the device limit; SA_EUNSUPPORTED for D != 64.
 * num_tokens = 0 does nothing and accepts null pointers.
 */
sa_status_t qkv_bias_rope(const void *qkv, const void *bias, const int32_t *positions,
                          const float *cos_sin, int64_t num_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t table_rows, void *q,
                          void *k, void *v, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_EPILOGUE_H */
