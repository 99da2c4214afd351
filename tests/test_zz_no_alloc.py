"""The decode entry point that allocates nothing (``sink_attn_decode_noalloc``), called
through the C ABI: its output equals the oracle's and that of ``sink_attn_decode`` with
proportional blocks and a caller workspace, to the bf16 bar, on two calls in a row (the
second with a smaller batch and shorter sequences, so the fixed state array holds the
first call's states when the second starts)."""
from __future__ import annotations

import ctypes
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


def noalloc_call(dev, q=None, cu_k=None, max_lk=None):
    """One sink_attn_decode_noalloc call straight through ctypes, into guarded outputs."""
    wl = dev.wl
    q = dev.q if q is None else q
    cu_k = dev.cu_k if cu_k is None else cu_k
    max_lk = dev.max_lk if max_lk is None else max_lk
    batch = cu_k.numel() - 1
    out, obuf = H.guarded((batch, wl.num_q_heads, wl.head_dim), dev.dtype)
    lse, lbuf = H.guarded((batch, wl.num_q_heads), torch.float32)
    lib = sa.load_library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    status = lib.sink_attn_decode_noalloc(
        sa.SA_BF16 if dev.bf16 else sa.SA_FP32, p(q), p(dev.k), p(dev.v), p(dev.sinks), p(cu_k),
        batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, max_lk, wl.sm_scale, p(out), p(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == sa.SA_OK, lib.sink_attn_last_error().decode()
    torch.cuda.synchronize()
    H.check_guard(obuf, out.numel())
    H.check_guard(lbuf, lse.numel())
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_decode_twice(dtype):
    orc = oracle.default()
    bf16 = dtype == "bf16"
    big = W.random_case(801, dtype=dtype, batch=12, hq=64, hkv=8, max_k=20000, decode=True,
                        sink_values=([-np.inf, 20.0, -20.0, 0.5] * 16))
    small = W.random_case(802, dtype=dtype, batch=3, hq=64, hkv=8, max_k=3000, decode=True)
    for wl in (big, small):  # the second call is the smaller one
        dev = H.Device(wl)
        ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
        out, lse = noalloc_call(dev)
        H.assert_close(out, ref, bf16=bf16)
        H.assert_lse_close(lse, ref_lse, bf16=bf16)
        wout, wlse = H.run_decode_call(dev, 0)
        H.assert_close(out, wout, bf16=bf16, what="noalloc vs workspace decode")
        H.assert_lse_close(lse, wlse, bf16=bf16)


def test_noalloc_ragged_long_decode():
    """The long-context ragged decode (8 sequences of 1024-131072 keys), every output."""
    orc = oracle.default()
    wl = W.workload(4)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    for _ in range(2):
        out, lse = noalloc_call(dev)
        H.assert_close(out, ref, bf16=True)
        H.assert_lse_close(lse, ref_lse, bf16=True)
    wout, _ = H.run_decode_call(dev, 0)
    H.assert_close(out, wout, bf16=True, what="noalloc vs workspace decode")
