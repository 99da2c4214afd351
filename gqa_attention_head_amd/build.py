"""Build the HIP library ``libsinkattn.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libsinkattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 vector ops are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)
    return res.returncode, msgs


def build(output: str = LIBRARY, verbose: bool = False, extra=()) -> str:
    """Compile every source under csrc/ into one shared library (always recompiles).

    Each source is compiled to an object in parallel, then the objects are linked."""
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS, *extra]
    tmp = output + ".tmp"
    with tempfile.TemporaryDirectory() as work:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(work, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *flags, "-c", "-o", obj, src])
        cmds.append([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds) - 1, os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, cmds[:-1]))
        results.append(_run(cmds[-1]) if all(rc == 0 for rc, _ in results) else (1, ""))
        for (rc, msgs), c in zip(results, cmds):
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}): {' '.join(c)}\n{msgs}")
            if msgs.strip() and verbose:
                print(msgs, file=sys.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
