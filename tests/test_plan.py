"""The proportional-block decode plan (kv_chunk_size = 0 in sink_attn_decode) checked on
the host: tests/plan/plan_check.cpp includes the library's own csrc/kernels.h, is built
with g++ and runs its invariants over 20000 seeded random batches (see that file)."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_attention_head_amd", "csrc")


def test_proportional_plan_invariants(tmp_path):
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers not installed")
    exe = str(tmp_path / "plan_check")
    build = subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__",
                            "-I/opt/rocm/include", "-I" + CSRC, "-o", exe,
                            os.path.join(ROOT, "tests", "plan", "plan_check.cpp")],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "cases" in run.stdout and int(run.stdout.split()[0]) > 15000
