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
