"""SINK_ATTN_DEBUG=1 checks the device-resident preconditions before any launch:
decreasing sequence offsets, lengths above the max_seqlen_* bounds, L_q > L_k under
causal masking and a +inf or NaN sink come back as SA_EINVAL, and valid calls still
run.  Runs in a child process, since the switch is read once per process."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import torch, gqa_attention_head_amd as sa
dev = "cuda"
q = torch.zeros(8, 8, 64, device=dev, dtype=torch.bfloat16)
k = torch.zeros(8, 1, 64, device=dev, dtype=torch.bfloat16)
s = torch.zeros(8, device=dev)
cu = lambda *x: torch.tensor(x, dtype=torch.int32, device=dev)
def code(fn):
    try:
        fn(); torch.cuda.synchronize(); return 0
    except sa.SinkAttnError as e:
        return e.status
res = {}
res["ok"] = code(lambda: sa.prefill(q, k, k, s, cu(0, 4, 8), cu(0, 4, 8), 4, 4, 0.125))
res["decreasing"] = code(lambda: sa.prefill(q, k, k, s, cu(0, 6, 4), cu(0, 6, 8), 6, 6, 0.125))
res["too_long"] = code(lambda: sa.prefill(q, k, k, s, cu(0, 4, 8), cu(0, 4, 8), 3, 4, 0.125))
res["causal_lq_gt_lk"] = code(lambda: sa.prefill(q, k, k, s, cu(0, 4, 8), cu(0, 2, 8), 4, 6, 0.125))
bad = s.clone(); bad[3] = float("inf")
res["inf_sink"] = code(lambda: sa.prefill(q, k, k, bad, cu(0, 4, 8), cu(0, 4, 8), 4, 4, 0.125))
nan = s.clone(); nan[0] = float("nan")
res["nan_sink_decode"] = code(lambda: sa.decode(q[:2].contiguous(), k, k, nan, cu(0, 4, 8), 4, 2, 0.125))
res["decode_too_long"] = code(lambda: sa.decode(q[:2].contiguous(), k, k, s, cu(0, 6, 8), 4, 2, 0.125))
res["decode_ok"] = code(lambda: sa.decode(q[:2].contiguous(), k, k, s, cu(0, 4, 8), 4, 2, 0.125))
print(res)
'''


def test_debug_mode_rejects_broken_device_inputs():
    env = dict(os.environ, SINK_ATTN_DEBUG="1", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True,
                         timeout=300, env=env)
    assert out.returncode == 0, out.stderr[-2000:]
    res = eval(out.stdout.strip().splitlines()[-1])
    EINVAL = 1
    assert res["ok"] == 0 and res["decode_ok"] == 0, res
    for key in ("decreasing", "too_long", "causal_lq_gt_lk", "inf_sink", "nan_sink_decode",
                "decode_too_long"):
        assert res[key] == EINVAL, (key, res)
