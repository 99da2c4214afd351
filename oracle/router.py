"""Top-K-then-softmax expert routing in fp64 (numpy).

TEST INFRASTRUCTURE ONLY.  The tests and the benchmark's CPU leg use it; the
product never imports it, and the two share no code.

"GPT-OSS on day 0" (Perplexity), MoE section: the gpt-oss router takes the
softmax over the top-K selected experts only (not over all experts, as some
DeepSeek-style routers do), and the expert weights are produced in bf16.  Read
here as: for each token, the K experts with the largest router logits (larger
first; equal logits ranked by lower expert index), and the softmax of those K
logits.  This function returns the weights in fp64; the device path rounds its
float32 weights to bf16, which the tests allow for.
"""
from __future__ import annotations

import numpy as np


def topk_softmax(logits, k: int):
    """logits: [T, E] array of the exact (finite) logit values; 1 <= k <= E.

    Returns (indices int32 [T, k], weights float64 [T, k]), experts in rank order.
    """
    z = np.asarray(logits, dtype=np.float64)
    if z.ndim != 2:
        raise ValueError("logits must be [T, E]")
    t, e = z.shape
    if not 1 <= k <= e:
        raise ValueError(f"k must be in [1, {e}]")
    expert = np.broadcast_to(np.arange(e), z.shape)
    # rank: larger logit first, then lower expert index (lexsort: last key is primary)
    order = np.lexsort((expert, -z), axis=-1)
    idx = order[:, :k]
    sel = np.take_along_axis(z, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])  # sel[:, 0] is the largest selected logit
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w
