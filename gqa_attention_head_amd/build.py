"""Build the HIP library ``libsinkattn.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

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


def build(output: str = LIBRARY, verbose: bool = False, extra=()) -> str:
    """Compile every source under csrc/ into one shared library (always recompiles)."""
    tmp = output + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS,
           *extra, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, file=sys.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
