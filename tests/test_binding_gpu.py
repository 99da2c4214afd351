"""GPU behaviour of the binding's convenience paths: prepared calls (``prepare_prefill``,
``prepare_decode``) re-issue exactly the call they were made from, over whatever the
tensors hold at the time; ``decode_noalloc`` through the binding matches the fp64
oracle.  Each result is also compared with the oracle."""
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


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_prepared_prefill_repeats_the_call(orc):
    """A prepared prefill gives the plain call's output bit for bit, and after the
    inputs are rewritten in place it computes over the new contents."""
    wl = W.random_case(501, batch=5, hq=16, hkv=2, max_q=200, max_k=400)
    dev = H.Device(wl)
    total_q = int(wl.cu_q[-1])
    out = torch.empty(total_q, wl.num_q_heads, wl.head_dim, dtype=dev.dtype, device="cuda")
    lse = torch.empty(total_q, wl.num_q_heads, dtype=torch.float32, device="cuda")
    call = sa.prepare_prefill(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q, dev.cu_k, dev.max_lq,
                              dev.max_lk, wl.sm_scale, out, causal=wl.causal, lse=lse)
    plain, plain_lse = H.run_prefill(dev)
    out.zero_()
    assert call() is out
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), plain) and np.array_equal(_np(lse), plain_lse)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(_np(out), ref, bf16=True)
    H.assert_lse_close(_np(lse), ref_lse, bf16=True)
    # new contents, same tensors: the prepared call follows them
    dev.q.mul_(-0.5), dev.k.mul_(2.0), dev.v.mul_(-1.0)
    call()
    torch.cuda.synchronize()
    again, again_lse = H.run_prefill(dev)
    assert np.array_equal(_np(out), again) and np.array_equal(_np(lse), again_lse)
    assert not np.array_equal(again, plain)


@pytest.mark.parametrize("chunk", [512, 0])
def test_prepared_decode_repeats_the_call(orc, chunk):
    """A prepared decode (fixed chunks, and proportional blocks) equals the plain call
    bit for bit and the oracle within the bf16 bar; it follows in-place input changes."""
    wl = W.random_case(503 + chunk, batch=9, hq=64, hkv=8, max_k=5000, decode=True)
    dev = H.Device(wl)
    slots = -(-dev.max_lk // chunk) if chunk else sa.balanced_slots(wl.batch, wl.num_q_heads, 64)
    ws = sa.DecodeWorkspace(wl.batch, wl.num_q_heads, slots, 64)
    out = torch.empty(wl.batch, wl.num_q_heads, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.batch, wl.num_q_heads, dtype=torch.float32, device="cuda")
    call = sa.prepare_decode(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk,
                             wl.sm_scale, ws, out, lse)
    out.zero_()
    call()
    plain, plain_lse = sa.decode(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk,
                                 wl.sm_scale, workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), _np(plain)) and np.array_equal(_np(lse), _np(plain_lse))
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(_np(out), ref, bf16=True)
    H.assert_lse_close(_np(lse), ref_lse, bf16=True)
    dev.q.mul_(-1.0)
    call()
    again = sa.decode(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk, wl.sm_scale,
                      workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(_np(out), _np(again))
    assert not np.array_equal(_np(out), _np(plain))


def test_decode_noalloc_through_the_binding(orc):
    """``sa.decode_noalloc`` (states in the library's fixed device array) against the
    oracle, twice in a row with a smaller batch the second time."""
    for seed, batch in ((505, 12), (506, 3)):
        wl = W.random_case(seed, batch=batch, hq=64, hkv=8, max_k=9000, decode=True)
        dev = H.Device(wl)
        out, lse = sa.decode_noalloc(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk,
                                     wl.sm_scale, return_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
        H.assert_close(_np(out), ref, bf16=True)
        H.assert_lse_close(_np(lse), ref_lse, bf16=True)
