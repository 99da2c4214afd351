"""Shared helpers for the GPU parity tests: upload a workload, call the HIP
library through its Python binding, compare against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import gqa_attention_head_amd as sa

# Tolerances on `out` against the fp64 oracle.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
FP32_MAX_ABS = 1e-5
# Diagnostic tolerance on the natural-log normaliser.
BF16_LSE, FP32_LSE = 1e-3, 1e-5
GUARD = 1024  # guard elements on each side of an output buffer


def to_device(arr: np.ndarray, bf16: bool) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


class Device:
    """A workload's tensors on the GPU."""

    def __init__(self, wl):
        self.wl = wl
        self.bf16 = wl.dtype == "bf16"
        q, k, v = wl.device_arrays()
        self.q = to_device(q, self.bf16)
        self.k = to_device(k, self.bf16)
        self.v = to_device(v, self.bf16)
        self.sinks = torch.from_numpy(wl.sinks).cuda()
        self.cu_q = torch.from_numpy(wl.cu_q).cuda()
        self.cu_k = torch.from_numpy(wl.cu_k).cuda()
        self.max_lq = int(wl.seqlens_q.max()) if wl.batch else 0
        self.max_lk = int(wl.seqlens_k.max()) if wl.batch else 0

    @property
    def dtype(self):
        return torch.bfloat16 if self.bf16 else torch.float32


def guarded(shape, dtype, fill=float("nan")):
    """An output tensor carved out of a larger buffer poisoned with `fill`.

    Returns (view, buffer); check_guard(buffer, view.numel()) verifies that no
    element outside the view was written."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device="cuda")
    return buf[GUARD:GUARD + n].view(*shape), buf


def check_guard(buf, n):
    head = buf[:GUARD].float().cpu().numpy()
    tail = buf[GUARD + n:].float().cpu().numpy()
    assert np.all(np.isnan(head)) and np.all(np.isnan(tail)), "write outside the output buffer"


def run_prefill(dev: Device, causal=None, lse=True):
    wl = dev.wl
    total_q = int(wl.cu_q[-1])
    out, obuf = guarded((total_q, wl.num_q_heads, wl.head_dim), dev.dtype)
    lse_t, lbuf = guarded((total_q, wl.num_q_heads), torch.float32)
    sa.prefill(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q, dev.cu_k, dev.max_lq, dev.max_lk,
               wl.sm_scale, causal=wl.causal if causal is None else causal, out=out,
               lse=lse_t if lse else None, return_lse=False)
    torch.cuda.synchronize()
    check_guard(obuf, out.numel())
    if lse:
        check_guard(lbuf, lse_t.numel())
    return out.float().cpu().numpy().astype(np.float64), (lse_t.cpu().numpy().astype(np.float64) if lse else None)


def run_decode(dev: Device, chunk: int, q=None, cu_k=None, max_lk=None, return_partials=False):
    """Split + merge for single-query sequences (q: [B, Hq, D])."""
    wl = dev.wl
    q = dev.q if q is None else q
    cu_k = dev.cu_k if cu_k is None else cu_k
    max_lk = dev.max_lk if max_lk is None else max_lk
    batch = cu_k.numel() - 1
    nch = max(1, -(-max_lk // chunk))
    pm, pd, pa = sa.partial_buffers(batch, wl.num_q_heads, nch, wl.head_dim)
    pm.fill_(float("nan")), pd.fill_(float("nan")), pa.fill_(float("nan"))
    sa.decode_split(q, dev.k, dev.v, dev.sinks, cu_k, max_lk, chunk, nch, wl.sm_scale,
                    partials=(pm, pd, pa))
    out, obuf = guarded((batch, wl.num_q_heads, wl.head_dim), dev.dtype)
    lse_t, lbuf = guarded((batch, wl.num_q_heads), torch.float32)
    sa.merge(pm, pd, pa, cu_k, chunk, out=out, lse=lse_t)
    torch.cuda.synchronize()
    check_guard(obuf, out.numel())
    check_guard(lbuf, lse_t.numel())
    res = (out.float().cpu().numpy().astype(np.float64), lse_t.cpu().numpy().astype(np.float64))
    if return_partials:
        res = res + (pm.cpu().numpy(), pd.cpu().numpy(), pa.cpu().numpy())
    return res


def assert_close(got, want, bf16: bool, what="out"):
    """Element-wise comparison to the tolerances stated above."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    if bf16:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max abs err {err.max():.3e} > {BF16_MAX_ABS}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs err {err.mean():.3e} > {BF16_MEAN_ABS}"
    else:
        assert err.max() <= FP32_MAX_ABS, f"{what}: max abs err {err.max():.3e} > {FP32_MAX_ABS}"
    return float(err.max()), float(err.mean())


def assert_lse_close(got, want, bf16: bool):
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), "lse: -inf pattern differs"
    assert np.all(got[~fin] == want[~fin])
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        tol = BF16_LSE if bf16 else FP32_LSE
        assert err <= tol, f"lse: max abs err {err:.3e} > {tol}"


def run_decode_call(dev: Device, chunk: int, q=None, cu_k=None, max_lk=None, workspace=None,
                     max_num_chunks=None):
    """One ``sink_attn_decode`` call (split pass and merge enqueued together)."""
    wl = dev.wl
    q = dev.q if q is None else q
    cu_k = dev.cu_k if cu_k is None else cu_k
    max_lk = dev.max_lk if max_lk is None else max_lk
    batch = cu_k.numel() - 1
    out, obuf = guarded((batch, wl.num_q_heads, wl.head_dim), dev.dtype)
    lse_t, lbuf = guarded((batch, wl.num_q_heads), torch.float32)
    sa.decode(q, dev.k, dev.v, dev.sinks, cu_k, max_lk, chunk, wl.sm_scale,
              max_num_chunks=max_num_chunks, workspace=workspace, out=out, lse=lse_t)
    torch.cuda.synchronize()
    check_guard(obuf, out.numel())
    check_guard(lbuf, lse_t.numel())
    return out.float().cpu().numpy().astype(np.float64), lse_t.cpu().numpy().astype(np.float64)
