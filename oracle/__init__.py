"""ctypes binding for the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product (``gqa_attention_head_amd``) never
imports it, and the two share no code.

The oracle implements attention with a per-head sink as stated in
"GPT-OSS on day 0" (Perplexity), section "Kernels for GPT-OSS / Sink
attention"; see ``oracle.c`` for the reading of that section.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

_F = ctypes.POINTER(ctypes.c_float)
_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Build the oracle with gcc (C11, OpenMP, -O2; no fast-math: IEEE double throughout)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return output


def _ptr(a, typ):
    return a.ctypes.data_as(typ) if a is not None else None


class Oracle:
    """Thin wrapper over one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [_F, _F, _F, _F, _I32, _I32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                         _I64, ctypes.c_int64, _D, _D, ctypes.c_int]
        lib.oracle_attention_split.restype = ctypes.c_int
        lib.oracle_attention_split.argtypes = [_F, _F, _F, _F, _I32, _I32, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_double, ctypes.c_int, ctypes.c_int64,
                                               _I64, ctypes.c_int64, _D, _D, ctypes.c_int]
        lib.oracle_partials.restype = ctypes.c_int
        lib.oracle_partials.argtypes = [_F, _F, _F, _F, _I32, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_int64, ctypes.c_int64, _D, _D, _D, ctypes.c_int]
        lib.oracle_split_row.restype = ctypes.c_int
        lib.oracle_split_row.argtypes = [_F, _F, _F, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_double, _I64, ctypes.c_int,
                                         _D, _D]
        self.lib = lib

    @staticmethod
    def _prep(q, k, v, sinks, cu_q, cu_k):
        f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
        i = lambda a: np.ascontiguousarray(a, dtype=np.int32)
        return f(q), f(k), f(v), f(sinks), i(cu_q), i(cu_k)

    def attention(self, q, k, v, sinks, cu_q, cu_k, sm_scale, causal=True, rows=None,
                  nthreads=None, chunk=None):
        """Direct definition (``chunk=None``) or the block-split method (``chunk`` keys).

        q: [total_q, Hq, D], k/v: [total_k, Hkv, D] float arrays holding the exact values.
        Returns (out [nrows, Hq, D] float64, lse [nrows, Hq] float64).
        """
        q, k, v, sinks, cu_q, cu_k = self._prep(q, k, v, sinks, cu_q, cu_k)
        batch = cu_q.shape[0] - 1
        hq, d = q.shape[1], q.shape[2]
        hkv = k.shape[1]
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows.shape[0]
        else:
            nrows = int(cu_q[-1] - cu_q[0])
        out = np.zeros((nrows, hq, d), dtype=np.float64)
        lse = np.zeros((nrows, hq), dtype=np.float64)
        nthreads = nthreads or (os.cpu_count() or 1)
        common = (_ptr(q, _F), _ptr(k, _F), _ptr(v, _F), _ptr(sinks, _F), _ptr(cu_q, _I32),
                  _ptr(cu_k, _I32), batch, hq, hkv, d, float(sm_scale), int(bool(causal)))
        if chunk is None:
            rc = self.lib.oracle_attention(*common, _ptr(rows, _I64), nrows, _ptr(out, _D),
                                           _ptr(lse, _D), int(nthreads))
        else:
            rc = self.lib.oracle_attention_split(*common, int(chunk), _ptr(rows, _I64), nrows,
                                                 _ptr(out, _D), _ptr(lse, _D), int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle returned {rc}")
        return out, lse

    def partials(self, q, k, v, sinks, cu_k, sm_scale, chunk, max_blocks, nthreads=None):
        """Per-block (m, d, acc) of single-query sequences (q: [B, Hq, D])."""
        q, k, v, sinks, _, cu_k = self._prep(q, k, v, sinks, np.zeros(1), cu_k)
        batch = cu_k.shape[0] - 1
        hq, d = q.shape[1], q.shape[2]
        hkv = k.shape[1]
        m = np.full((batch, hq, max_blocks), np.nan)
        dd = np.full((batch, hq, max_blocks), np.nan)
        acc = np.full((batch, hq, max_blocks, d), np.nan)
        rc = self.lib.oracle_partials(_ptr(q, _F), _ptr(k, _F), _ptr(v, _F), _ptr(sinks, _F),
                                      _ptr(cu_k, _I32), batch, hq, hkv, d, float(sm_scale),
                                      int(chunk), int(max_blocks), _ptr(m, _D), _ptr(dd, _D),
                                      _ptr(acc, _D), int(nthreads or (os.cpu_count() or 1)))
        if rc != 0:
            raise ValueError(f"oracle returned {rc}")
        return m, dd, acc

    def split_row(self, qrow, keys, values, sm_scale, sink, bounds):
        """One query against keys [n, D] and values [n, D] over an explicit key partition."""
        qrow = np.ascontiguousarray(qrow, dtype=np.float32)
        keys = np.ascontiguousarray(keys, dtype=np.float32).reshape(-1, qrow.shape[0])
        values = np.ascontiguousarray(values, dtype=np.float32).reshape(-1, qrow.shape[0])
        bounds = np.ascontiguousarray(bounds, dtype=np.int64)
        d = qrow.shape[0]
        out = np.zeros(d, dtype=np.float64)
        lse = np.zeros(1, dtype=np.float64)
        rc = self.lib.oracle_split_row(_ptr(qrow, _F), _ptr(keys, _F), _ptr(values, _F), d,
                                       keys.shape[0], d, float(sm_scale), float(sink),
                                       _ptr(bounds, _I64), bounds.shape[0] - 1, _ptr(out, _D),
                                       _ptr(lse, _D))
        if rc != 0:
            raise ValueError(f"oracle returned {rc}")
        return out, float(lse[0])

    def workload(self, wl, rows=None, nthreads=None, chunk=None):
        """Run on a :class:`gqa_attention_head_amd.workloads.Workload`."""
        return self.attention(wl.q32, wl.k32, wl.v32, wl.sinks, wl.cu_q, wl.cu_k, wl.sm_scale,
                              causal=wl.causal, rows=rows, nthreads=nthreads, chunk=chunk)


_DEFAULT = None


def default(rebuild: bool = False) -> Oracle:
    """The oracle built from ``oracle.c`` next to this file (compiled on first use), or
    the library that SINK_ATTN_ORACLE_LIBRARY names (the sanitizer build of the tests)."""
    global _DEFAULT
    override = os.environ.get("SINK_ATTN_ORACLE_LIBRARY")
    if override:
        if _DEFAULT is None or _DEFAULT.path != override:
            _DEFAULT = Oracle(override)
        return _DEFAULT
    if _DEFAULT is None or rebuild:
        if rebuild or not os.path.exists(LIBRARY) or \
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            compile_library()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def build_variant(source_text: str, directory: str | None = None) -> Oracle:
    """Compile an edited copy of the oracle source (used by tests that plant a mistake)."""
    directory = directory or tempfile.mkdtemp(prefix="oracle_variant_")
    src = os.path.join(directory, "oracle_variant.c")
    with open(src, "w") as f:
        f.write(source_text)
    return Oracle(compile_library(src, os.path.join(directory, "liboracle_variant.so")))
