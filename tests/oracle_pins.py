"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` when the oracle disagrees with what the mathematics or the
pages fix.  ``tests/test_oracle.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in a copy of the
oracle source and checks that some pin catches each one.

What is pinned ("GPT-OSS on day 0", Perplexity, section "Kernels for GPT-OSS /
Sink attention", unless stated):
  * sink = -inf gives ordinary softmax attention (torch's fp64 CPU attention
    with an explicit bottom-right causal mask);
  * the sink is one extra softmax entry with a zero value vector
    (torch.softmax over the scores with the sink appended);
  * closed forms: one key, L identical keys, no keys, the effect of the sink
    as an exact scaling of the sink-free output, hand-worked fixtures;
  * the blocked online method (running max seeded with the sink in the first
    block only, log-sum-exp combine) equals the direct definition for every
    block length and every contiguous partition of the keys;
  * grouped-query head mapping (query head h reads KV head h / G);
  * a prefill row equals a decode of the same query over its visible keys;
  * the per-block partial states equal attention over that block alone.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

from gqa_attention_head_amd.workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = dict(rtol=1e-10, atol=1e-12)


def _case(seed, lq, lk, hq=4, hkv=2, d=16, causal=True, sinks=None, dtype="fp32"):
    return make_workload(f"pin{seed}", dtype=dtype, kind="prefill", seqlens_q=lq, seqlens_k=lk,
                         num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=seed, causal=causal,
                         sink_values=sinks)


def _torch_attention(wl, extra_sink: bool):
    """Library attention per sequence in fp64 on the CPU.

    extra_sink=False: torch scaled_dot_product_attention with an explicit
    bottom-right boolean mask (the sink is ignored).
    extra_sink=True: torch.softmax over [scores | sink] and the product with
    [V ; 0], i.e. the sink as one more key whose value is zero.
    """
    g = wl.num_q_heads // wl.num_kv_heads
    outs = []
    for b in range(wl.batch):
        q = torch.from_numpy(wl.q32[wl.cu_q[b]:wl.cu_q[b + 1]]).double().permute(1, 0, 2)
        k = torch.from_numpy(wl.k32[wl.cu_k[b]:wl.cu_k[b + 1]]).double().permute(1, 0, 2)
        v = torch.from_numpy(wl.v32[wl.cu_k[b]:wl.cu_k[b + 1]]).double().permute(1, 0, 2)
        k = k.repeat_interleave(g, dim=0).contiguous()
        v = v.repeat_interleave(g, dim=0).contiguous()
        lq, lk = q.shape[1], k.shape[1]
        i = torch.arange(lq)[:, None]
        j = torch.arange(lk)[None, :]
        mask = (j <= lk - lq + i) if wl.causal else torch.ones(lq, lk, dtype=torch.bool)
        if not extra_sink:
            o = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None], v[None], attn_mask=mask[None, None], scale=wl.sm_scale)[0]
        else:
            s = torch.matmul(q, k.transpose(1, 2).contiguous()) * wl.sm_scale
            s = s.masked_fill(~mask[None], -math.inf)
            sink = torch.from_numpy(wl.sinks).double()[:, None, None].expand(-1, lq, 1)
            p = torch.softmax(torch.cat([s, sink], dim=2), dim=2)
            vz = torch.cat([v, torch.zeros(v.shape[0], 1, v.shape[2], dtype=v.dtype)], dim=1)
            o = torch.matmul(p, vz)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


def pin_sink_neg_inf_is_softmax(orc):
    """sink = -inf: ordinary GQA softmax attention, causal bottom-right and non-causal."""
    for causal in (True, False):
        wl = _case(11, [5, 17, 1, 33], [9, 17, 40, 50], hq=6, hkv=2, d=8, causal=causal,
                   sinks=[-np.inf] * 6)
        out, _ = orc.workload(wl, nthreads=2)
        ref = _torch_attention(wl, extra_sink=False)
        np.testing.assert_allclose(out, ref, **TIGHT)


def pin_extra_key_identity(orc):
    """The sink is one more softmax entry with value vector 0."""
    wl = _case(12, [7, 20, 3], [7, 31, 64], hq=8, hkv=2, d=16,
               sinks=[-3.0, -0.5, 0.0, 0.7, 1.5, 4.0, 9.0, -np.inf])
    out, _ = orc.workload(wl, nthreads=2)
    ref = _torch_attention(wl, extra_sink=True)
    np.testing.assert_allclose(out, ref, **TIGHT)


def _single_query(orc, keys, values, qvec, sink, sm_scale=1.0):
    """Decode-shaped call: one query, one head, keys/values [n, D]."""
    n, d = keys.shape
    q = np.asarray(qvec, dtype=np.float32).reshape(1, 1, d)
    k = np.asarray(keys, dtype=np.float32).reshape(n, 1, d)
    v = np.asarray(values, dtype=np.float32).reshape(n, 1, d)
    if n == 0:
        k = np.zeros((0, 1, d), dtype=np.float32)
        v = np.zeros((0, 1, d), dtype=np.float32)
    out, lse = orc.attention(q, k, v, np.array([sink], dtype=np.float32),
                             np.array([0, 1]), np.array([0, n]), sm_scale, causal=False,
                             nthreads=1)
    return out[0, 0], lse[0, 0]


def pin_closed_forms(orc):
    rng = np.random.default_rng(13)
    d = 8
    for sink in (-2.0, 0.0, 0.375, 5.0):  # exactly representable in float32
        # one key: out = sigmoid(s - sink) v, lse = logaddexp(s, sink)
        qv = rng.standard_normal(d).astype(np.float32)
        kv = rng.standard_normal((1, d)).astype(np.float32)
        vv = rng.standard_normal((1, d)).astype(np.float32)
        s = 0.25 * float(np.dot(qv.astype(np.float64), kv[0].astype(np.float64)))
        out, lse = _single_query(orc, kv, vv, qv, sink, sm_scale=0.25)
        sig = 1.0 / (1.0 + math.exp(sink - s))
        np.testing.assert_allclose(out, sig * vv[0].astype(np.float64), **TIGHT)
        np.testing.assert_allclose(lse, np.logaddexp(s, sink), **TIGHT)
        # L identical keys and values: out = v L e^s / (L e^s + e^sink)
        for L in (2, 7, 40):
            keys = np.repeat(kv, L, axis=0)
            vals = np.repeat(vv, L, axis=0)
            out, lse = _single_query(orc, keys, vals, qv, sink, sm_scale=0.25)
            w = L * math.exp(s) / (L * math.exp(s) + math.exp(sink))
            np.testing.assert_allclose(out, w * vv[0].astype(np.float64), **TIGHT)
            np.testing.assert_allclose(lse, math.log(L * math.exp(s) + math.exp(sink)), **TIGHT)
    # no keys: out = 0; lse = sink, or -inf when the sink is -inf too
    out, lse = _single_query(orc, np.zeros((0, d)), np.zeros((0, d)), np.ones(d), 1.5)
    assert np.all(out == 0.0) and lse == 1.5
    out, lse = _single_query(orc, np.zeros((0, d)), np.zeros((0, d)), np.ones(d), -np.inf)
    assert np.all(out == 0.0) and lse == -np.inf


def pin_sink_scaling(orc):
    """A finite sink scales the sink-free output by 1 / (1 + e^(sink - lse0)) exactly,
    so the output shrinks monotonically toward 0 as the sink grows (large-sink limit)."""
    wl0 = _case(14, [9, 1], [9, 300], hq=4, hkv=1, d=16, sinks=[-np.inf] * 4)
    out0, lse0 = orc.workload(wl0, nthreads=2)
    prev = None
    for sink in (-5.0, 0.0, 3.0, 20.0, 40.0):
        wl = _case(14, [9, 1], [9, 300], hq=4, hkv=1, d=16, sinks=[sink] * 4)
        out, lse = orc.workload(wl, nthreads=2)
        scale = 1.0 / (1.0 + np.exp(sink - lse0))
        np.testing.assert_allclose(out, out0 * scale[..., None], **TIGHT)
        np.testing.assert_allclose(lse, np.logaddexp(lse0, sink), **TIGHT)
        mag = np.abs(out).max()
        if prev is not None:
            assert mag < prev
        prev = mag
    # sink = +20 with N(0,1) scores: |out| <= max|v| * sum e^s / (sum e^s + e^20)
    bound = np.abs(wl0.v32).max() / (1.0 + np.exp(20.0 - lse0))
    wl = _case(14, [9, 1], [9, 300], hq=4, hkv=1, d=16, sinks=[20.0] * 4)
    out, _ = orc.workload(wl, nthreads=2)
    assert np.all(np.abs(out) <= bound[..., None] * (1 + 1e-12))


def pin_split_invariance(orc):
    """The blocked method equals the direct definition for every block length."""
    wl = _case(15, [1, 23, 41], [1, 37, 41], hq=4, hkv=2, d=8,
               sinks=[-np.inf, -1.0, 0.5, 6.0])
    ref, ref_lse = orc.workload(wl, nthreads=2)
    for chunk in range(1, 42):
        out, lse = orc.workload(wl, chunk=chunk, nthreads=2)
        np.testing.assert_allclose(out, ref, **TIGHT)
        np.testing.assert_allclose(lse, ref_lse, **TIGHT)


def pin_brute_force_partitions(orc):
    """Tiny inputs: every contiguous partition of the keys (sink in the first part)
    agrees with the unshifted extended-precision e^s / (e^sink + sum e^s)."""
    rng = np.random.default_rng(16)
    for L in range(0, 9):
        d = int(rng.integers(1, 5))
        qv = rng.standard_normal(d).astype(np.float32)
        keys = rng.standard_normal((L, d)).astype(np.float32)
        vals = rng.standard_normal((L, d)).astype(np.float32)
        sink = float(np.float32(rng.standard_normal()))
        sm = 0.5
        s = [np.longdouble(sm) * sum(np.longdouble(qv[t]) * np.longdouble(keys[j, t])
                                     for t in range(d)) for j in range(L)]
        e = [np.exp(x) for x in s]
        z = np.exp(np.longdouble(sink)) + sum(e, np.longdouble(0))
        want = np.array([sum((e[j] * np.longdouble(vals[j, t]) for j in range(L)),
                             np.longdouble(0)) / z for t in range(d)], dtype=np.float64)
        want_lse = float(np.log(z))
        cuts = range(1, L)
        for r in range(0, max(L, 1)):
            for chosen in itertools.combinations(cuts, r):
                bounds = [0, *chosen, L]
                out, lse = orc.split_row(qv, keys, vals, sm, sink, bounds)
                np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
                np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-14)


def pin_gqa_mapping(orc):
    """Query head h reads KV head h // G: same result as multi-head attention
    over K/V repeated G times along the head axis."""
    wl = _case(17, [6, 11], [6, 30], hq=8, hkv=2, d=8)
    out, lse = orc.workload(wl, nthreads=2)
    g = wl.num_q_heads // wl.num_kv_heads
    out2, lse2 = orc.attention(wl.q32, np.repeat(wl.k32, g, axis=1), np.repeat(wl.v32, g, axis=1),
                               wl.sinks, wl.cu_q, wl.cu_k, wl.sm_scale, causal=True, nthreads=2)
    np.testing.assert_allclose(out, out2, **TIGHT)
    np.testing.assert_allclose(lse, lse2, **TIGHT)


def pin_prefill_equals_decode(orc):
    """Causal row i of a sequence (Lq queries over Lk keys) equals a single-query
    call over the first Lk - Lq + i + 1 keys."""
    wl = _case(18, [12], [29], hq=4, hkv=1, d=8)
    out, lse = orc.workload(wl, nthreads=2)
    lq, lk = 12, 29
    for i in range(lq):
        n = lk - lq + i + 1
        o, l = orc.attention(wl.q32[i:i + 1], wl.k32[:n], wl.v32[:n], wl.sinks,
                             np.array([0, 1]), np.array([0, n]), wl.sm_scale, causal=False,
                             nthreads=1)
        np.testing.assert_allclose(out[i], o[0], **TIGHT)
        np.testing.assert_allclose(lse[i], l[0], **TIGHT)


def pin_partials(orc):
    """Block c's state (m, d, acc) normalises to attention over block c's keys alone,
    with the sink present in block 0 only."""
    wl = make_workload("pin_partials", dtype="fp32", kind="decode", seqlens_q=[1, 1, 1],
                       seqlens_k=[50, 7, 0], num_q_heads=4, num_kv_heads=2, head_dim=8, seed=19,
                       causal=False, sink_values=[-1.0, 0.0, 2.0, -np.inf])
    chunk, nb = 16, 4
    m, dd, acc = orc.partials(wl.q32, wl.k32, wl.v32, wl.sinks, wl.cu_k, wl.sm_scale, chunk, nb,
                              nthreads=2)
    for b in range(wl.batch):
        lk = int(wl.seqlens_k[b])
        for c in range(max(1, -(-lk // chunk))):
            lo, hi = c * chunk, min((c + 1) * chunk, lk)
            ks = wl.k32[wl.cu_k[b] + lo:wl.cu_k[b] + hi]
            vs = wl.v32[wl.cu_k[b] + lo:wl.cu_k[b] + hi]
            sinks = wl.sinks if c == 0 else np.full_like(wl.sinks, -np.inf)
            o, l = orc.attention(wl.q32[b:b + 1], ks, vs, sinks, np.array([0, 1]),
                                 np.array([0, hi - lo]), wl.sm_scale, causal=False, nthreads=1)
            for h in range(wl.num_q_heads):
                if l[0, h] == -np.inf:
                    assert m[b, h, c] == -np.inf
                    continue
                np.testing.assert_allclose(acc[b, h, c] / dd[b, h, c], o[0, h], **TIGHT)
                np.testing.assert_allclose(m[b, h, c] + np.log(dd[b, h, c]), l[0, h], **TIGHT)


def pin_golden(orc):
    """Hand-worked examples stored under tests/golden/."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float32)
        d = q.shape[2]
        k = np.array(c["k"], dtype=np.float32).reshape(-1, c.get("hkv", 1), d)
        v = np.array(c["v"], dtype=np.float32).reshape(-1, c.get("hkv", 1), d)
        sinks = np.array([float(x) for x in c["sinks"]], dtype=np.float32)
        out, lse = orc.attention(q, k, v, sinks, np.array(c["cu_q"]), np.array(c["cu_k"]),
                                 c["sm_scale"], causal=c["causal"], nthreads=1)
        np.testing.assert_allclose(out, np.array(c["out"], dtype=np.float64), rtol=1e-12,
                                   atol=1e-12)
        want_lse = np.array([[float(x) for x in row] for row in c["lse"]], dtype=np.float64)
        np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


ALL_PINS = [
    pin_sink_neg_inf_is_softmax,
    pin_extra_key_identity,
    pin_closed_forms,
    pin_sink_scaling,
    pin_split_invariance,
    pin_brute_force_partitions,
    pin_gqa_mapping,
    pin_prefill_equals_decode,
    pin_partials,
    pin_golden,
]
