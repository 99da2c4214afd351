"""GPU parity of per-row attention states written to a chosen slot
(sink_attn_prefill_state) and of cascade attention built from them: new tokens of
several sequences attend a shared cached prefix in one call and their own keys in
another, and sink_attn_merge_rows combines the two slots.  The oracle is the plain
definition over each sequence's concatenated keys (prefix, then its own keys), with
bottom-right causal masking."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import gqa_attention_head_amd as sa
from gqa_attention_head_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

import gpu_helpers as H  # noqa: E402

NTHREADS = min(16, os.cpu_count() or 1)
D = 64


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def draw(rng, shape, bf16):
    x = rng.standard_normal(shape, dtype=np.float32)
    if bf16:
        bits = W.bf16_round(x)
        return W.bf16_widen(bits), bits
    return x, None


def dev_tensor(vals, bits, bf16):
    return H.to_device(bits if bf16 else vals, bf16)


def cu(lengths):
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lengths)
    return out


def states_to_out(pm, pd, pa, slot):
    m = pm[..., slot].cpu().numpy().astype(np.float64)
    d = pd[..., slot].cpu().numpy().astype(np.float64)
    acc = pa[..., slot, :].cpu().numpy().astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(d[..., None] > 0, acc / d[..., None], 0.0)
        lse = np.where(d > 0, m + np.log(d), -np.inf)
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("group", [8, 3])
@pytest.mark.parametrize("include_sink", [True, False])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_state_slot(orc, dtype, group, include_sink, causal):
    """One call's states land in the chosen slot only (the others keep their poison)
    and normalise to the oracle's attention over that call's keys, with the sink or
    with none (sink = -inf)."""
    bf16 = dtype == "bf16"
    rng = np.random.default_rng(81 + group)
    hkv = 2
    hq = hkv * group
    lq, lk = [70, 1, 33], [200, 64, 33]
    q32, q16 = draw(rng, (sum(lq), hq, D), bf16)
    k32, k16 = draw(rng, (sum(lk), hkv, D), bf16)
    v32, v16 = draw(rng, (sum(lk), hkv, D), bf16)
    sinks = rng.standard_normal(hq).astype(np.float32)
    sinks[0] = -np.inf
    cu_q, cu_k = cu(lq), cu(lk)
    q, k, v = (dev_tensor(a, b, bf16) for a, b in ((q32, q16), (k32, k16), (v32, v16)))
    num_slots, slot = 3, 1
    parts = sa.partial_buffers(sum(lq), hq, num_slots, D)
    for t in parts:
        t.fill_(float("nan"))
    pm, pd, pa = sa.prefill_state(q, k, v, torch.from_numpy(sinks).cuda(),
                                  torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(),
                                  max(lq), max(lk), 0.125, causal=causal,
                                  include_sink=include_sink, slot=slot, partials=parts)
    torch.cuda.synchronize()
    for t in (pm, pd, pa):
        others = torch.cat([t[:, :, s] .reshape(-1) for s in range(num_slots) if s != slot])
        assert torch.isnan(others).all(), "a slot other than the chosen one was written"
    out, lse = states_to_out(pm, pd, pa, slot)
    ref_sinks = sinks if include_sink else np.full(hq, -np.inf, np.float32)
    ref, ref_lse = orc.attention(q32, k32, v32, ref_sinks, cu_q, cu_k, 0.125, causal=causal,
                                 nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=bf16)
    H.assert_lse_close(lse, ref_lse, bf16=bf16)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("group", [8, 4, 3, 32])
def test_cascade_shared_prefix(orc, dtype, group):
    """Shared prefix of 1000 keys, four sequences with 1..300 new tokens each: the
    prefix call (all new tokens as one non-causal row block, sink included) and the
    per-sequence causal call (no sink), merged, equal attention over prefix + own
    keys."""
    bf16 = dtype == "bf16"
    rng = np.random.default_rng(90 + group)
    hkv = 2
    hq = hkv * group
    prefix, new = 1000, [300, 1, 77, 129]
    total = sum(new)
    q32, q16 = draw(rng, (total, hq, D), bf16)
    kp32, kp16 = draw(rng, (prefix, hkv, D), bf16)
    vp32, vp16 = draw(rng, (prefix, hkv, D), bf16)
    ks32, ks16 = draw(rng, (total, hkv, D), bf16)
    vs32, vs16 = draw(rng, (total, hkv, D), bf16)
    sinks = (2.0 * rng.standard_normal(hq)).astype(np.float32)
    sinks[1] = -np.inf
    q = dev_tensor(q32, q16, bf16)
    kp, vp = dev_tensor(kp32, kp16, bf16), dev_tensor(vp32, vp16, bf16)
    ks, vs = dev_tensor(ks32, ks16, bf16), dev_tensor(vs32, vs16, bf16)
    s_d = torch.from_numpy(sinks).cuda()
    parts = sa.partial_buffers(total, hq, 2, D)
    # shared prefix: every new token of every sequence, one row block, sink included
    sa.prefill_state(q, kp, vp, s_d, torch.tensor([0, total], dtype=torch.int32, device="cuda"),
                     torch.tensor([0, prefix], dtype=torch.int32, device="cuda"), total, prefix,
                     0.125, causal=False, include_sink=True, slot=0, partials=parts)
    # each sequence's own keys, causal, no sink
    cu_new = torch.from_numpy(cu(new)).cuda()
    sa.prefill_state(q, ks, vs, s_d, cu_new, cu_new, max(new), max(new), 0.125, causal=True,
                     include_sink=False, slot=1, partials=parts)
    out, lse = sa.merge_rows(*parts, out_dtype=q.dtype, return_lse=True)
    torch.cuda.synchronize()
    # oracle: each sequence's keys are the prefix followed by its own keys
    kf = np.concatenate(sum(([kp32, ks32[a:b]] for a, b in zip(cu(new)[:-1], cu(new)[1:])), []))
    vf = np.concatenate(sum(([vp32, vs32[a:b]] for a, b in zip(cu(new)[:-1], cu(new)[1:])), []))
    ref, ref_lse = orc.attention(q32, kf, vf, sinks, cu(new), cu([prefix + n for n in new]),
                                 0.125, causal=True, nthreads=NTHREADS)
    H.assert_close(out.float().cpu().numpy().astype(np.float64), ref, bf16=bf16)
    H.assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, bf16=bf16)
