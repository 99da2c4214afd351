"""Pre-attention epilogue in fp64 (numpy): QKV bias add and rotary embedding.

TEST INFRASTRUCTURE ONLY.  The tests and the benchmark's CPU leg use it; the
product never imports it, and the two share no code.

"GPT-OSS on day 0" (Perplexity), architecture list: the QKV projections carry
biases, and positions are encoded with YaRN rotary embeddings (as in
DeepSeek-V3).  The YaRN frequencies and its attention scale are folded into a
per-position table (row p: cos(p theta_i) for i < D/2, then sin(p theta_i),
both already multiplied by the scale), so this function only applies it:

    x = qkv + bias                                   (per token, all heads)
    q, k heads:  y_i       = x_i c_i - x_{i+D/2} s_i
                 y_{i+D/2} = x_{i+D/2} c_i + x_i s_i     (i < D/2; rotate halves)
    v heads:     y = x
"""
from __future__ import annotations

import numpy as np


def qkv_bias_rope(qkv, bias, positions, cos_sin, hq: int, hkv: int, d: int = 64):
    """qkv: [T, (hq + 2 hkv) * d]; bias: [(hq + 2 hkv) * d]; positions: [T] ints;
    cos_sin: [rows, d].  Positions outside [0, rows) take the nearest row.
    Returns q [T, hq, d], k [T, hkv, d], v [T, hkv, d] in float64."""
    x = np.asarray(qkv, dtype=np.float64) + np.asarray(bias, dtype=np.float64)[None, :]
    t = x.shape[0]
    x = x.reshape(t, hq + 2 * hkv, d)
    rows = np.asarray(cos_sin, dtype=np.float64)
    pos = np.clip(np.asarray(positions, dtype=np.int64), 0, rows.shape[0] - 1)
    c = rows[pos, : d // 2][:, None, :]
    s = rows[pos, d // 2:][:, None, :]
    qk = x[:, : hq + hkv]
    lo, hi = qk[..., : d // 2], qk[..., d // 2:]
    rot = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
    return rot[:, :hq], rot[:, hq:], x[:, hq + hkv:]
