"""CPU sanitizer leg: the fp64 oracle (oracle/oracle.c) and the C ABI's host-side
argument validation (csrc/api.cpp with the host-only capability table) built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal, then exercised by
the oracle pins and by the ABI rejection tests in subprocesses that preload the
sanitizer runtime.  The kernels and the HIP runtime are replaced by host stubs that
report no device (tests/sanitizer/host_stubs.cpp), so nothing here needs a GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_attention_head_amd", "csrc")
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-g", "-O1", "-fPIC", "-shared"]


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not path or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitized")
    oracle_lib, abi_lib = str(d / "liboracle_san.so"), str(d / "libsinkattn_host_san.so")
    _build(["gcc", "-std=c11", "-fopenmp", *FLAGS, "-o", oracle_lib,
            os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    _build(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            f"-I{ROOT}/include", f"-I{CSRC}", *FLAGS, "-o", abi_lib,
            os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "capabilities.cpp"),
            os.path.join(ROOT, "tests", "sanitizer", "host_stubs.cpp")])
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT,
               SINK_ATTN_ORACLE_LIBRARY=oracle_lib, SINK_ATTN_LIBRARY=abi_lib, OMP_NUM_THREADS="4")
    return env, d


def _pytest(env, *args):
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           *args], capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)


@pytest.mark.parametrize("body,report", [
    # one element past a heap block
    ("unsigned *a = calloc(n, sizeof(unsigned)); unsigned s = 0;"
     " for (int i = 0; i <= n; ++i) s += a[i]; free(a); return (int)s;", "heap-buffer-overflow"),
    # signed overflow
    ("int s = 0x7ffffff0; for (int i = 0; i < n; ++i) s += 8; return s;", "signed integer overflow"),
])
def test_sanitizers_catch_a_planted_mistake(sanitized, body, report):
    """The harness itself: a mistake planted in a library built the same way must end
    the subprocess with the sanitizer's report."""
    env, d = sanitized
    src, lib = d / "planted.c", str(d / "libplanted.so")
    src.write_text("#include <stdlib.h>\nint planted(int n) { " + body + " }\n")
    _build(["gcc", "-std=c11", *FLAGS, "-o", lib, str(src)])
    code = f"import ctypes; ctypes.CDLL({lib!r}).planted(8)"
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120)
    assert res.returncode != 0
    assert report in res.stderr


def test_oracle_pins_under_sanitizers(sanitized):
    env, _ = sanitized
    res = _pytest(env, "tests/test_oracle.py")
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout


def test_abi_validation_under_sanitizers(sanitized):
    env, _ = sanitized
    res = _pytest(env, "tests/test_abi.py")
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout
