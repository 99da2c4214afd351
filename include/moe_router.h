/*
 * moe_router.h -- C ABI of the expert-routing step of a mixture-of-experts
 * layer, in the same library as sink_attn.h (libsinkattn.so, gfx950).
 *
 * "GPT-OSS on day 0" (Perplexity), MoE section: the gpt-oss router takes the
 * softmax over the top-K selected experts only (not over all experts), and the
 * expert weights are computed in bf16.  Read here as: for every token, the K
 * experts with the largest router logits, ranked larger logit first and equal
 * logits by lower expert index, and the softmax of those K logits, computed in
 * float32 from the bf16 logits and rounded to bf16 (round to nearest even).
 */
#ifndef MOE_ROUTER_H
#define MOE_ROUTER_H

#include <stdint.h>

#include "sink_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * logits   [num_tokens, num_experts] bf16, device pointer, 16-byte aligned, finite
 *          values (NaN and infinities are outside the contract)
 * indices  [num_tokens, k] int32, device pointer (written): experts in rank order
 * weights  [num_tokens, k] bf16, device pointer (written): softmax of the k
 *          selected logits, in the same order
 * num_experts in {8, 16, 32, 64, 128, 256, 512}; 1 <= k <= min(8, num_experts).
 * The caller owns every buffer; the call is asynchronous on `stream`.
 * Errors: SA_EINVAL for num_tokens < 0, k out of range or (with num_tokens > 0)
 * null pointers or misaligned logits; SA_EUNSUPPORTED for another num_experts; SA_ELAUNCH for launch
 * failures.  num_tokens = 0 does nothing and accepts null pointers.
 */
sa_status_t moe_topk_softmax(const void *logits, int64_t num_tokens, int32_t num_experts,
                             int32_t k, int32_t *indices, void *weights, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTER_H */
