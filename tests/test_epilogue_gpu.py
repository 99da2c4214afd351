"""GPU parity of the pre-attention epilogue (qkv_bias_rope) against the fp64 oracle.

The kernel adds the bias and rotates in float32 and rounds once to bf16, so each
output is within half a bf16 step of its float32 value (2^-9 relative, 2^-8 allowed)
plus the float32 error of the bias sum and the two-term rotation, at most a few
2^-24 of |x_i c_i| + |x_{i+32} s_i| (2^-21 allowed)."""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_head_amd as sa
from gqa_attention_head_amd import workloads as W
from oracle.rope import qkv_bias_rope as ref_rope

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

from gpu_helpers import check_guard, guarded  # noqa: E402

D = 64


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def widen(t):
    return W.bf16_widen(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def bound(qkv32, bias32, pos, table, hq, hkv):
    """Per-element error allowance: 2^-8 |y| + 2^-21 (|x_i c_i| + |x_{i+32} s_i|) on the
    rotated heads, 2^-8 |y| + 2^-21 |x| on the value heads."""
    t = qkv32.shape[0]
    x = (qkv32.astype(np.float64) + bias32.astype(np.float64)[None]).reshape(t, hq + 2 * hkv, D)
    p = np.clip(pos.astype(np.int64), 0, table.shape[0] - 1)
    c = np.abs(table[p, : D // 2].astype(np.float64))[:, None]
    s = np.abs(table[p, D // 2:].astype(np.float64))[:, None]
    ax = np.abs(x[:, : hq + hkv])
    lo, hi = ax[..., : D // 2], ax[..., D // 2:]
    mag = np.concatenate([lo * c + hi * s, hi * c + lo * s], axis=-1)
    return mag[:, :hq], mag[:, hq:], np.abs(x[:, hq + hkv:])


def check(got, ref, mag):
    err = np.abs(got - ref)
    lim = 2.0 ** -8 * np.abs(ref) + 2.0 ** -21 * mag
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (bad[:5], err[tuple(bad[0])], lim[tuple(bad[0])])


def run_case(seed, tokens, hq, hkv, max_pos=8192, positions=None, rows=None):
    qkv16, qkv32, b16, b32, pos, table = W.qkv_epilogue_inputs(seed, tokens, hq, hkv, D, max_pos)
    if positions is not None:
        pos = positions.astype(np.int32)
    print(f"qkv_bias_rope seed={seed} T={tokens} Hq={hq} Hkv={hkv} rows={table.shape[0]}", flush=True)
    q, qbuf = guarded((tokens, hq, D), torch.bfloat16)
    k, kbuf = guarded((tokens, hkv, D), torch.bfloat16)
    v, vbuf = guarded((tokens, hkv, D), torch.bfloat16)
    sa.qkv_bias_rope(bf16_dev(qkv16), bf16_dev(b16), torch.from_numpy(pos).cuda(),
                     torch.from_numpy(table).cuda(), hq, hkv, q=q, k=k, v=v)
    torch.cuda.synchronize()
    for buf, n in ((qbuf, q.numel()), (kbuf, k.numel()), (vbuf, v.numel())):
        check_guard(buf, n)
    sel = slice(None) if rows is None else rows
    rq, rk, rv = ref_rope(qkv32[sel], b32, pos[sel], table, hq, hkv, D)
    mq, mk, mv = bound(qkv32[sel], b32, pos[sel], table, hq, hkv)
    check(widen(q)[sel], rq, mq)
    check(widen(k)[sel], rk, mk)
    check(widen(v)[sel], rv, mv)
    return rq, rk, rv


@pytest.mark.parametrize("tokens,hq,hkv", [
    (1, 1, 1), (3, 8, 1), (37, 8, 2), (300, 64, 8), (513, 12, 4), (97, 5, 3), (129, 64, 1),
])
def test_epilogue_cases(tokens, hq, hkv):
    run_case(tokens * 100 + hq + hkv, tokens, hq, hkv, max_pos=512)


def test_epilogue_positions_outside_the_table_take_the_nearest_row():
    tokens, rows = 64, 100
    pos = np.array([-(1 << 30), -5, -1, 0, 1, 99, 100, 101, 1 << 30] * 8)[:tokens]
    pos = np.concatenate([pos, np.arange(tokens - pos.size)]).astype(np.int32)
    run_case(7, tokens, 8, 1, max_pos=rows, positions=pos)


def test_epilogue_position_zero_is_bias_only():
    """Row 0 of the table is (scale, ..., scale, 0, ..., 0): q and k are the biased
    input times the YaRN attention scale, v the biased input (bf16-rounded)."""
    tokens, hq, hkv = 40, 8, 2
    rq, rk, _ = run_case(8, tokens, hq, hkv, max_pos=64, positions=np.zeros(tokens, np.int32))
    _, qkv32, _, b32, _, table = W.qkv_epilogue_inputs(8, tokens, hq, hkv, D, 64)
    x = (qkv32.astype(np.float64) + b32[None]).reshape(tokens, hq + 2 * hkv, D)
    np.testing.assert_allclose(rq, x[:, :hq] * table[0, 0], rtol=1e-12)


def test_epilogue_large_sampled():
    """16384 tokens x (64 + 2 x 8) heads, the size the benchmark runs; checked on a
    seeded sample of 512 tokens (the guards and the rest of the layout on all)."""
    tokens = 16384
    rows = np.sort(np.random.default_rng(11).choice(tokens, 512, replace=False))
    run_case(11, tokens, 64, 8, max_pos=8192, rows=rows)


def test_epilogue_empty():
    z = torch.empty(0, (8 + 4) * D, device="cuda", dtype=torch.bfloat16)
    b = torch.zeros((8 + 4) * D, device="cuda", dtype=torch.bfloat16)
    q, k, v = sa.qkv_bias_rope(z, b, torch.empty(0, device="cuda", dtype=torch.int32),
                               torch.ones(4, D, device="cuda"), 8, 2)
    torch.cuda.synchronize()
    assert q.shape == (0, 8, D) and k.shape == (0, 2, D) and v.shape == (0, 2, D)


def test_epilogue_feeds_prefill():
    """Epilogue then causal sink prefill, against the oracle's epilogue rounded to bf16
    then the oracle's attention: the bf16 attention bar."""
    import oracle
    from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS
    hq, hkv, lens = 16, 2, [200, 77, 1]
    tokens = sum(lens)
    qkv16, qkv32, b16, b32, _, table = W.qkv_epilogue_inputs(21, tokens, hq, hkv, D, 4096)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    sinks = np.random.default_rng(21).standard_normal(hq).astype(np.float32)
    q, k, v = sa.qkv_bias_rope(bf16_dev(qkv16), bf16_dev(b16), torch.from_numpy(pos).cuda(),
                               torch.from_numpy(table).cuda(), hq, hkv)
    cu_d = torch.from_numpy(cu).cuda()
    out = sa.prefill(q, k, v, torch.from_numpy(sinks).cuda(), cu_d, cu_d, max(lens), max(lens),
                        sm_scale=0.125, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = ref_rope(qkv32, b32, pos, table, hq, hkv, D)
    r16 = [W.bf16_widen(W.bf16_round(a.astype(np.float32))) for a in (rq, rk, rv)]
    ref, _ = oracle.default().attention(*r16, sinks, cu, cu, 0.125, causal=True)
    err = np.abs(widen(out) - ref)
    assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS, (err.max(), err.mean())
