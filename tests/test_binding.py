"""Host-side behaviour of the Python binding and bench.py on a machine without a
GPU: every entry point refuses host tensors before touching the library's kernels,
and bench.py refuses more than one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

import gqa_attention_head_amd as sa  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(sa.LIBRARY):
        from gqa_attention_head_amd import build
        build.build()


def host(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_prefill_refuses_host_tensors():
    q, k = host(4, 8, 64), host(4, 2, 64)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        sa.prefill(q, k, k, host(8, dtype=torch.float32), cu, cu, 4, 4, 0.125)


def test_decode_and_split_entry_points_refuse_host_tensors():
    q, k = host(2, 8, 64), host(8, 2, 64)
    s = host(8, dtype=torch.float32)
    cu = torch.tensor([0, 4, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        sa.decode_split(q, k, k, s, cu, 4, 2, 2, 0.125)
    with pytest.raises(ValueError, match="device tensor"):
        sa.prefill_split(q, k, k, s, cu, cu, 4, 4, 2, 0.125)
    with pytest.raises(ValueError, match="device tensor"):
        sa.prefill_state(q, k, k, s, cu, cu, 4, 4, 0.125, num_slots=2)


def test_router_and_epilogue_refuse_host_tensors():
    with pytest.raises(ValueError, match="device tensor"):
        sa.topk_softmax(host(16, 128), 4)
    with pytest.raises(ValueError, match="device tensor"):
        sa.qkv_bias_rope(host(3, 12 * 64), host(12 * 64), torch.zeros(3, dtype=torch.int32),
                         host(8, 64, dtype=torch.float32), 8, 2)


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, PYTHONPATH=ROOT))
    assert res.returncode == 2
    assert "one GPU" in res.stderr


# ------------------------------------------------------------------ shape checks
# Every mis-shaped argument is refused with ValueError before the library is called
# and before the device check, so these run on host tensors; the library is replaced
# by a stand-in that fails the test if any of its functions is reached.

class NoLibrary:
    """Stands in for the loaded library: any call into it fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"library function {name} reached with a mis-shaped argument")


@pytest.fixture()
def no_library(monkeypatch):
    monkeypatch.setattr(sa, "_lib", NoLibrary())
    yield


def _qkv(tq=6, hq=8, hkv=2, d=64, tk=10):
    return host(tq, hq, d), host(tk, hkv, d), host(tk, hkv, d), host(hq, dtype=torch.float32)


def _cu(*xs):
    return torch.tensor(xs, dtype=torch.int32)


@pytest.mark.parametrize("case", [
    "sinks_len", "head_dim", "kv_shape", "cu_len", "out_shape", "lse_shape", "dims", "dtype_mix"])
def test_prefill_rejects_mis_shaped(no_library, case):
    q, k, v, s = _qkv()
    cq, ck = _cu(0, 2, 6), _cu(0, 4, 10)
    kw = {}
    if case == "sinks_len":
        s = host(7, dtype=torch.float32)
    elif case == "head_dim":
        k, v = host(10, 2, 32), host(10, 2, 32)
    elif case == "kv_shape":
        v = host(9, 2, 64)
    elif case == "cu_len":
        ck = _cu(0, 10)
    elif case == "out_shape":
        kw["out"] = host(6, 8, 32)
    elif case == "lse_shape":
        kw["lse"] = host(6, 7, dtype=torch.float32)
    elif case == "dims":
        q = host(6, 8 * 64)
    elif case == "dtype_mix":
        k = host(10, 2, 64, dtype=torch.float32)
    with pytest.raises((ValueError, TypeError)):
        sa.prefill(q, k, v, s, cq, ck, 4, 6, 0.125, **kw)


@pytest.mark.parametrize("case", ["partials", "sinks_len", "cu_len"])
def test_prefill_split_rejects_mis_shaped(no_library, case):
    q, k, v, s = _qkv()
    cq, ck = _cu(0, 2, 6), _cu(0, 4, 10)
    parts = None
    if case == "partials":
        parts = (host(6, 8, 3, dtype=torch.float32), host(6, 8, 3, dtype=torch.float32),
                 host(6, 8, 2, 64, dtype=torch.float32))  # acc holds 2 slots, m and d 3
    elif case == "sinks_len":
        s = host(16, dtype=torch.float32)
    elif case == "cu_len":
        cq = _cu(0, 6)
    with pytest.raises(ValueError):
        sa.prefill_split(q, k, v, s, cq, ck, 4, 6, 2, 0.125, max_num_chunks=3, partials=parts)


@pytest.mark.parametrize("case", ["rows", "slots_arg", "acc_dim"])
def test_prefill_state_rejects_mis_shaped(no_library, case):
    q, k, v, s = _qkv()
    cq, ck = _cu(0, 2, 6), _cu(0, 4, 10)
    f = dict(dtype=torch.float32)
    parts = (host(6, 8, 2, **f), host(6, 8, 2, **f), host(6, 8, 2, 64, **f))
    kw = dict(partials=parts)
    if case == "rows":
        kw["partials"] = (host(5, 8, 2, **f), host(5, 8, 2, **f), host(5, 8, 2, 64, **f))
    elif case == "slots_arg":
        kw["num_slots"] = 3
    elif case == "acc_dim":
        kw["partials"] = (parts[0], parts[1], host(6, 8, 2, 32, **f))
    with pytest.raises(ValueError):
        sa.prefill_state(q, k, v, s, cq, ck, 4, 6, 0.125, **kw)


@pytest.mark.parametrize("case", ["out", "lse", "d_slots", "acc_rank"])
def test_merge_rows_rejects_mis_shaped(no_library, case):
    f = dict(dtype=torch.float32)
    pm, pd, pa = host(5, 8, 3, **f), host(5, 8, 3, **f), host(5, 8, 3, 64, **f)
    kw = {}
    if case == "out":
        kw["out"] = host(5, 8, 32)
    elif case == "lse":
        kw["lse"] = host(5, 4, **f)
    elif case == "d_slots":
        pd = host(5, 8, 4, **f)
    elif case == "acc_rank":
        pa = host(5, 8, 3 * 64, **f)
    with pytest.raises(ValueError):
        sa.merge_rows(pm, pd, pa, **kw)


@pytest.mark.parametrize("case", ["q_batch", "partials", "sinks_len", "head_dim"])
def test_decode_split_rejects_mis_shaped(no_library, case):
    q, k, v, s = _qkv(tq=2)
    cu = _cu(0, 4, 10)
    f = dict(dtype=torch.float32)
    parts = None
    if case == "q_batch":
        q = host(3, 8, 64)
    elif case == "partials":
        parts = (host(2, 8, 2, **f), host(2, 8, 2, **f), host(2, 8, 2, 64, **f))  # 3 slots asked
    elif case == "sinks_len":
        s = host(4, dtype=torch.float32)
    elif case == "head_dim":
        q = host(2, 8, 128)
    with pytest.raises(ValueError):
        sa.decode_split(q, k, v, s, cu, 6, 2, 3, 0.125, partials=parts)


@pytest.mark.parametrize("case", ["batch", "out", "lse", "acc"])
def test_merge_rejects_mis_shaped(no_library, case):
    f = dict(dtype=torch.float32)
    pm, pd, pa = host(2, 8, 3, **f), host(2, 8, 3, **f), host(2, 8, 3, 64, **f)
    cu = _cu(0, 4, 10)
    kw = {}
    if case == "batch":
        cu = _cu(0, 4, 10, 12)
    elif case == "out":
        kw["out"] = host(2, 8, 63)
    elif case == "lse":
        kw["lse"] = host(2, 9, **f)
    elif case == "acc":
        pa = host(2, 8, 2, 64, **f)
    with pytest.raises(ValueError):
        sa.merge(pm, pd, pa, cu, 2, **kw)


class _Workspace:
    def __init__(self, batch, hq, slots, d=64):
        f = dict(dtype=torch.float32)
        self.batch, self.num_q_heads, self.head_dim, self.max_num_chunks = batch, hq, d, slots
        self.partials = (host(batch, hq, slots, **f), host(batch, hq, slots, **f),
                         host(batch, hq, slots, d, **f))


@pytest.mark.parametrize("case", ["ws_batch", "ws_heads", "ws_slots_arg", "ws_buffers", "out",
                                  "lse", "q_batch", "chunk"])
def test_decode_rejects_mis_shaped(no_library, case):
    q, k, v, s = _qkv(tq=2)
    cu = _cu(0, 4, 10)
    ws = _Workspace(2, 8, 3)
    kw = dict(workspace=ws)
    chunk = 2
    if case == "ws_batch":
        kw["workspace"] = _Workspace(3, 8, 3)
    elif case == "ws_heads":
        kw["workspace"] = _Workspace(2, 16, 3)
    elif case == "ws_slots_arg":
        kw["max_num_chunks"] = 5
    elif case == "ws_buffers":
        ws.partials = (ws.partials[0], ws.partials[1], host(2, 8, 2, 64, dtype=torch.float32))
    elif case == "out":
        kw["out"] = host(2, 8, 32)
    elif case == "lse":
        kw["lse"] = host(2, dtype=torch.float32)
    elif case == "q_batch":
        q = host(1, 8, 64)
    elif case == "chunk":
        chunk = -1
    with pytest.raises(ValueError):
        sa.decode(q, k, v, s, cu, 6, chunk, 0.125, **kw)


def test_decode_graph_rejects_mis_shaped(no_library):
    q, k, v, s = _qkv(tq=2)
    with pytest.raises(ValueError):
        sa.DecodeGraph(q, k, v, host(3, dtype=torch.float32), _cu(0, 4, 10), 6, 2, 0.125)
    with pytest.raises(ValueError):
        sa.DecodeGraph(q, k, v, s, _cu(0, 4, 10), 6, 2, 0.125, out=host(2, 8, 32))


@pytest.mark.parametrize("case", ["indices", "weights", "rank"])
def test_router_rejects_mis_shaped(no_library, case):
    logits = host(16, 128)
    kw = {}
    if case == "indices":
        kw["indices"] = torch.zeros(16, 3, dtype=torch.int32)
    elif case == "weights":
        kw["weights"] = host(15, 4)
    elif case == "rank":
        logits = host(16, 128, 1)
    with pytest.raises(ValueError):
        sa.topk_softmax(logits, 4, **kw)


@pytest.mark.parametrize("case", ["qkv", "bias", "positions", "table", "q_out"])
def test_epilogue_rejects_mis_shaped(no_library, case):
    args = dict(qkv=host(3, 12 * 64), bias=host(12 * 64), positions=torch.zeros(3, dtype=torch.int32),
                cos_sin=host(8, 64, dtype=torch.float32))
    kw = {}
    if case == "qkv":
        args["qkv"] = host(3, 11 * 64)
    elif case == "bias":
        args["bias"] = host(11 * 64)
    elif case == "positions":
        args["positions"] = torch.zeros(4, dtype=torch.int32)
    elif case == "table":
        args["cos_sin"] = host(8, 32, dtype=torch.float32)
    elif case == "q_out":
        kw["q"] = host(3, 7, 64)
    with pytest.raises(ValueError):
        sa.qkv_bias_rope(args["qkv"], args["bias"], args["positions"], args["cos_sin"], 8, 2, **kw)


def test_prepared_calls_and_noalloc_reject_mis_shaped(no_library):
    """prepare_prefill, prepare_decode and decode_noalloc run the same checks before any
    library call."""
    q, k, v, s = _qkv()
    cq, ck = _cu(0, 2, 6), _cu(0, 4, 10)
    with pytest.raises(ValueError):  # sinks of the wrong length
        sa.prepare_prefill(q, k, v, host(7, dtype=torch.float32), cq, ck, 4, 6, 0.125,
                           host(6, 8, 64))
    with pytest.raises(ValueError):  # out of the wrong head dim
        sa.prepare_prefill(q, k, v, s, cq, ck, 4, 6, 0.125, host(6, 8, 32))
    q, k, v, s = _qkv(tq=2)
    cu = _cu(0, 4, 10)
    with pytest.raises(ValueError):  # out of the wrong head dim
        sa.prepare_decode(q, k, v, s, cu, 6, 2, 0.125, _Workspace(2, 8, 3), host(2, 8, 32))
    with pytest.raises(ValueError):  # workspace for another batch
        sa.prepare_decode(q, k, v, s, cu, 6, 2, 0.125, _Workspace(3, 8, 3), host(2, 8, 64))
    with pytest.raises(ValueError):  # cu_seqlens_k for another batch
        sa.decode_noalloc(q, k, v, s, _cu(0, 4, 10, 12), 6, 0.125)
    with pytest.raises(ValueError):  # lse of the wrong shape
        sa.decode_noalloc(q, k, v, s, cu, 6, 0.125, lse=host(2, 9, dtype=torch.float32))
