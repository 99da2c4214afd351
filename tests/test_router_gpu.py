"""GPU parity of the top-K-then-softmax expert router (moe_topk_softmax) against
the fp64 oracle: expert indices bit for bit; each bf16 weight equal to the oracle's
weight rounded to bf16, or its neighbour (the float32 weight may fall on the other
side of a bf16 rounding boundary than the exact one)."""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_head_amd as sa
from gqa_attention_head_amd import workloads as W
from oracle.router import topk_softmax

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)


def run(bits, k):
    lg = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    idx, w = sa.topk_softmax(lg, k)
    torch.cuda.synchronize()
    wbits = w.view(torch.int16).cpu().numpy().view(np.uint16)
    return idx.cpu().numpy(), wbits


def check(bits, vals, k, rows=None):
    idx, wbits = run(bits, k)
    if rows is not None:
        idx, wbits, vals = idx[rows], wbits[rows], vals[rows]
    ref_idx, ref_w = topk_softmax(vals, k)
    assert np.array_equal(idx, ref_idx), np.argwhere(idx != ref_idx)[:5]
    ref_bits = W.bf16_round(ref_w.astype(np.float32)).astype(np.int32)
    gap = np.abs(wbits.astype(np.int32) - ref_bits)
    assert gap.max() <= 1, (gap.max(), np.argwhere(gap > 1)[:5])
    got = W.bf16_widen(wbits).astype(np.float64)
    assert np.abs(got.sum(axis=1) - 1.0).max() <= k * 2.0 ** -8


@pytest.mark.parametrize("experts", [8, 16, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("k", [1, 2, 4, 8])
@pytest.mark.parametrize("ties", [False, True])
def test_router_cases(experts, k, ties):
    if k > experts:
        pytest.skip("k > experts")
    tokens = 1000 + experts + k  # not a multiple of the tokens one wave step handles
    bits, vals = W.router_logits(experts * 10 + k, tokens, experts, ties=ties)
    check(bits, vals, k)


def test_router_k_equals_e_is_full_softmax():
    bits, vals = W.router_logits(5, 300, 8)
    check(bits, vals, 8)


def test_router_empty():
    lg = torch.empty(0, 128, device="cuda", dtype=torch.bfloat16)
    idx, w = sa.topk_softmax(lg, 4)
    assert idx.shape == (0, 4) and w.shape == (0, 4)


def test_router_large_sampled():
    """The benchmark's size (2^20 tokens, 128 experts, top-4), checked on sampled tokens."""
    bits, vals = W.router_logits(12, 1 << 20, 128)
    rows = np.random.default_rng(0).choice(1 << 20, 4096, replace=False)
    check(bits, vals, 4, rows=rows)
