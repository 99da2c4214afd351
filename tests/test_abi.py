"""C-ABI contract on the CPU: the library loads, exports what include/sink_attn.h
declares, and rejects invalid arguments before launching anything."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
import sys

import pytest

import gqa_attention_head_amd as sa
from gqa_attention_head_amd import build as sa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIBRARY):
        sa_build.build()
    return sa.load_library()


def declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b((?:sink_attn|moe|qkv)_\w+)\s*\(", text,
                                flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(sa.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


P = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first
NULL = None


def _prefill(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_q=P, cu_k=P, batch=2, hq=64, hkv=8,
             d=64, max_q=16, max_k=16, scale=0.125, causal=1, out=P, lse=NULL, stream=NULL)
    a.update(kw)
    return lib.sink_attn_prefill(*a.values())


def _split(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_k=P, batch=2, hq=64, hkv=8, d=64,
             max_k=4096, chunk=512, max_chunks=8, scale=0.125, pm=P, pd=P, pa=P, stream=NULL)
    a.update(kw)
    return lib.sink_attn_decode_split(*a.values())


def _decode(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_k=P, batch=2, hq=64, hkv=8, d=64,
             max_k=4096, chunk=512, max_chunks=8, scale=0.125, pm=P, pd=P, pa=P, out=P, lse=NULL, stream=NULL)
    a.update(kw)
    return lib.sink_attn_decode(*a.values())


def _prefill_split(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_q=P, cu_k=P, batch=2, hq=64, hkv=8,
             d=64, max_q=4096, max_k=4096, chunk=1024, max_chunks=4, scale=0.125, causal=1,
             pm=P, pd=P, pa=P, stream=NULL)
    a.update(kw)
    return lib.sink_attn_prefill_split(*a.values())


def _merge_rows(lib, **kw):
    a = dict(dtype=sa.SA_BF16, pm=P, pd=P, pa=P, rows=100, hq=64, d=64, max_chunks=4, out=P,
             lse=NULL, stream=NULL)
    a.update(kw)
    return lib.sink_attn_merge_rows(*a.values())


def _merge(lib, **kw):
    a = dict(dtype=sa.SA_BF16, pm=P, pd=P, pa=P, cu_k=P, chunk=512, max_chunks=8, batch=2,
             hq=64, d=64, out=P, lse=NULL, stream=NULL)
    a.update(kw)
    return lib.sink_attn_merge(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), sa.SA_EINVAL),
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(sinks=NULL), sa.SA_EINVAL),
    (dict(batch=0), sa.SA_EINVAL),
    (dict(hq=60, hkv=8), sa.SA_EINVAL),
    (dict(hkv=0), sa.SA_EINVAL),
    (dict(d=128), sa.SA_EUNSUPPORTED),
    (dict(hq=128, hkv=1), sa.SA_EUNSUPPORTED),
    (dict(dtype=7), sa.SA_EINVAL),
    (dict(causal=2), sa.SA_EINVAL),
    (dict(max_q=-1), sa.SA_EINVAL),
    (dict(scale=float("nan")), sa.SA_EINVAL),
    (dict(scale=0.0), sa.SA_EINVAL),
    (dict(scale=-0.125), sa.SA_EINVAL),
])
def test_prefill_rejects(lib, kw, status):
    assert _prefill(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(pa=NULL), sa.SA_EINVAL),
    (dict(chunk=0), sa.SA_EINVAL),            # proportional blocks: the one-call decode only
    (dict(max_chunks=7), sa.SA_EINVAL),       # ceil(4096 / 512) = 8 slots needed
    (dict(max_k=-1), sa.SA_EINVAL),
    (dict(hq=64, hkv=7), sa.SA_EINVAL),
    (dict(d=32), sa.SA_EUNSUPPORTED),
    (dict(scale=float("inf")), sa.SA_EINVAL),
    # chunk c starts at c * chunk in 32 bits: max_num_chunks * chunk must stay below 2^31
    (dict(chunk=1 << 20, max_chunks=2049, max_k=4096), sa.SA_EINVAL),
    (dict(chunk=0x7FFFFFFF, max_chunks=2, max_k=4096), sa.SA_EINVAL),
])
def test_decode_split_rejects(lib, kw, status):
    assert _split(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(pm=NULL), sa.SA_EINVAL),
    (dict(max_chunks=7), sa.SA_EINVAL),
    (dict(hq=64, hkv=5), sa.SA_EINVAL),
    (dict(d=96), sa.SA_EUNSUPPORTED),
    (dict(chunk=-1), sa.SA_EINVAL),
    (dict(chunk=0, max_chunks=0), sa.SA_EINVAL),        # proportional blocks need a slot
    (dict(chunk=1 << 20, max_chunks=2048, max_k=4096), sa.SA_EINVAL),  # chunk span past 2^31
])
def test_decode_rejects(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(chunk=0), sa.SA_EINVAL),
    (dict(max_chunks=0), sa.SA_EINVAL),
    (dict(batch=0), sa.SA_EINVAL),
    (dict(d=80), sa.SA_EUNSUPPORTED),
    (dict(chunk=1 << 28, max_chunks=8), sa.SA_EINVAL),  # chunk span past 2^31
])
def test_merge_rejects(lib, kw, status):
    assert _merge(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


# q, k, v and part_acc are moved in 16-byte pieces, a prefill out row in 8-byte pieces
MIS16 = ctypes.c_void_p(0x1000 + 8)   # 8-byte but not 16-byte aligned
MIS8 = ctypes.c_void_p(0x1000 + 4)


@pytest.mark.parametrize("call,kw", [
    (_prefill, dict(q=MIS16)), (_prefill, dict(k=MIS16)), (_prefill, dict(v=MIS16)),
    (_prefill, dict(out=MIS8)),
    (_prefill_split, dict(pa=MIS16)), (_prefill_split, dict(q=MIS16)),
    (_split, dict(k=MIS16)), (_split, dict(pa=MIS16)),
    (_decode, dict(v=MIS16)), (_decode, dict(pa=MIS16)),
])
def test_misaligned_pointers_rejected(lib, call, kw):
    assert call(lib, **kw) == sa.SA_EINVAL
    assert "aligned" in lib.sink_attn_last_error().decode()


def test_aligned_out_of_fp32_width_accepted_by_validation(lib):
    # an 8-byte-aligned prefill out passes the alignment check (it fails later only for
    # want of a device, or not at all with max_q = 0)
    assert _prefill(lib, out=ctypes.c_void_p(0x1000 + 8), max_q=0) == sa.SA_OK


def test_empty_prefill_is_a_no_op(lib):
    assert _prefill(lib, max_q=0) == sa.SA_OK


@pytest.mark.skipif(not _no_gpu(), reason="needs a host without a GPU (would launch on fake pointers)")
def test_valid_call_without_device_reports_launch_error(lib):
    assert _prefill(lib) == sa.SA_ELAUNCH
    assert "device" in lib.sink_attn_last_error().decode()
    assert _split(lib) == sa.SA_ELAUNCH
    assert _merge(lib) == sa.SA_ELAUNCH
    assert _decode(lib) == sa.SA_ELAUNCH
    # proportional blocks (chunk 0) pass validation with any slot count >= 1
    assert _decode(lib, chunk=0, max_chunks=1) == sa.SA_ELAUNCH
    assert _decode(lib, chunk=0, max_chunks=300) == sa.SA_ELAUNCH
    # the largest chunk span that fits: 2^31 - 1 keys in one chunk
    assert _split(lib, chunk=0x7FFFFFFF, max_chunks=1, max_k=4096) == sa.SA_ELAUNCH


def test_missing_library_fails_loudly(tmp_path):
    code = ("import gqa_attention_head_amd as sa\n"
            "try:\n    sa.load_library()\nexcept RuntimeError as e:\n    print('raised', e)\n")
    env = dict(os.environ, SINK_ATTN_LIBRARY=str(tmp_path / "absent.so"), PYTHONPATH=ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env)
    assert "raised" in res.stdout


def test_product_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "gqa_attention_head_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), fn
                assert "oracle.c" not in text and "liboracle" not in text, fn
    code = "import sys, gqa_attention_head_amd; print('oracle' in sys.modules)"
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         env=dict(os.environ, PYTHONPATH=ROOT), check=True)
    assert res.stdout.strip() == "False"


@pytest.mark.parametrize("kw,status", [
    (dict(pm=NULL), sa.SA_EINVAL),
    (dict(cu_q=NULL), sa.SA_EINVAL),
    (dict(chunk=0), sa.SA_EINVAL),
    (dict(max_chunks=3), sa.SA_EINVAL),        # ceil(4096 / 1024) = 4 slots needed
    (dict(causal=3), sa.SA_EINVAL),
    (dict(hq=64, hkv=6), sa.SA_EINVAL),
    (dict(d=80), sa.SA_EUNSUPPORTED),
    (dict(scale=0.0), sa.SA_EINVAL),
    (dict(dtype=sa.SA_FP32, batch=3000, max_chunks=40, max_k=40960), sa.SA_EINVAL),  # generic grid
    # chunk c starts at c * chunk in 32 bits: an over-provisioned chunk count whose
    # last chunk would start past 2^31 is refused (2049 slots of 2^20 keys)
    (dict(chunk=1 << 20, max_chunks=2049, max_k=4096), sa.SA_EINVAL),
])
def test_prefill_split_rejects(lib, kw, status):
    assert _prefill_split(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(pa=NULL), sa.SA_EINVAL),
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(rows=-1), sa.SA_EINVAL),
    (dict(hq=0), sa.SA_EINVAL),
    (dict(max_chunks=0), sa.SA_EINVAL),
    (dict(d=128), sa.SA_EUNSUPPORTED),
    (dict(dtype=5), sa.SA_EINVAL),
])
def test_merge_rows_rejects(lib, kw, status):
    assert _merge_rows(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


def test_split_entry_points_empty_work_needs_no_device(lib):
    """Zero query rows / zero merge rows are valid no-ops (no device touched)."""
    assert _prefill_split(lib, max_q=0) == sa.SA_OK
    assert _merge_rows(lib, rows=0) == sa.SA_OK


def _router(lib, **kw):
    a = dict(logits=P, tokens=1000, experts=128, k=4, idx=P, w=P, stream=NULL)
    a.update(kw)
    return lib.moe_topk_softmax(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(logits=NULL), sa.SA_EINVAL),
    (dict(idx=NULL), sa.SA_EINVAL),
    (dict(w=NULL), sa.SA_EINVAL),
    (dict(tokens=-1), sa.SA_EINVAL),
    (dict(k=0), sa.SA_EINVAL),
    (dict(k=9), sa.SA_EINVAL),
    (dict(experts=8, k=8), None),              # valid: checked below without a device
    (dict(experts=4, k=2), sa.SA_EUNSUPPORTED),
    (dict(experts=96), sa.SA_EUNSUPPORTED),
    (dict(experts=1024), sa.SA_EUNSUPPORTED),
    (dict(logits=ctypes.c_void_p(258)), sa.SA_EINVAL),  # not 16-byte aligned
])
def test_router_rejects(lib, kw, status):
    if status is None:
        assert _router(lib, tokens=0, **kw) == sa.SA_OK
        return
    assert _router(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


def _rope(lib, **kw):
    a = dict(qkv=P, bias=P, pos=P, cs=P, tokens=1000, hq=64, hkv=8, d=64, rows=4096, q=P, k=P,
             v=P, stream=NULL)
    a.update(kw)
    return lib.qkv_bias_rope(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=NULL), sa.SA_EINVAL),
    (dict(bias=NULL), sa.SA_EINVAL),
    (dict(pos=NULL), sa.SA_EINVAL),
    (dict(cs=NULL), sa.SA_EINVAL),
    (dict(v=NULL), sa.SA_EINVAL),
    (dict(tokens=-1), sa.SA_EINVAL),
    (dict(hq=0), sa.SA_EINVAL),
    (dict(hkv=0), sa.SA_EINVAL),
    (dict(rows=0), sa.SA_EINVAL),
    (dict(d=128), sa.SA_EUNSUPPORTED),
    (dict(k=ctypes.c_void_p(264)), sa.SA_EINVAL),   # not 16-byte aligned
    (dict(tokens=1 << 40), sa.SA_EINVAL),       # grid beyond 2^31 - 1 blocks
])
def test_qkv_bias_rope_rejects(lib, kw, status):
    assert _rope(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


def test_qkv_bias_rope_empty_is_a_no_op(lib):
    assert _rope(lib, tokens=0, qkv=NULL, q=NULL) == sa.SA_OK


def _state(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_q=P, cu_k=P, batch=2, hq=64, hkv=8,
             d=64, max_q=4096, max_k=4096, scale=0.125, causal=1, sink=1, slot=0, nslots=2,
             pm=P, pd=P, pa=P, stream=NULL)
    a.update(kw)
    return lib.sink_attn_prefill_state(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(pa=NULL), sa.SA_EINVAL),
    (dict(cu_k=NULL), sa.SA_EINVAL),
    (dict(sink=2), sa.SA_EINVAL),
    (dict(slot=2), sa.SA_EINVAL),
    (dict(slot=-1), sa.SA_EINVAL),
    (dict(nslots=0), sa.SA_EINVAL),
    (dict(causal=5), sa.SA_EINVAL),
    (dict(hq=64, hkv=6), sa.SA_EINVAL),
    (dict(d=128), sa.SA_EUNSUPPORTED),
    (dict(scale=float("nan")), sa.SA_EINVAL),
    (dict(dtype=9), sa.SA_EINVAL),
])
def test_prefill_state_rejects(lib, kw, status):
    assert _state(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


def test_prefill_state_empty_is_a_no_op(lib):
    assert _state(lib, max_q=0) == sa.SA_OK


def _probe(lib, **kw):
    a = dict(buf=P, nbytes=1 << 20, blocks=1024, out=P, stream=NULL)
    a.update(kw)
    return lib.sink_attn_read_probe(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(buf=NULL), sa.SA_EINVAL),
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(out=NULL, nbytes=0), sa.SA_EINVAL),
    (dict(nbytes=-16), sa.SA_EINVAL),
    (dict(nbytes=24), sa.SA_EINVAL),            # not a multiple of 16
    (dict(blocks=0), sa.SA_EINVAL),
    (dict(blocks=65536), sa.SA_EINVAL),
    (dict(buf=ctypes.c_void_p(264)), sa.SA_EINVAL),  # not 16-byte aligned
])
def test_read_probe_rejects(lib, kw, status):
    assert _probe(lib, **kw) == status
    assert lib.sink_attn_read_probe is not None and lib.sink_attn_last_error().decode()


def _noalloc(lib, **kw):
    a = dict(dtype=sa.SA_BF16, q=P, k=P, v=P, sinks=P, cu_k=P, batch=2, hq=64, hkv=8, d=64,
             max_k=4096, scale=0.125, out=P, lse=NULL, stream=NULL)
    a.update(kw)
    return lib.sink_attn_decode_noalloc(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), sa.SA_EINVAL),
    (dict(out=NULL), sa.SA_EINVAL),
    (dict(cu_k=NULL), sa.SA_EINVAL),
    (dict(max_k=-1), sa.SA_EINVAL),
    (dict(hq=64, hkv=6), sa.SA_EINVAL),
    (dict(d=128), sa.SA_EUNSUPPORTED),
    (dict(scale=0.0), sa.SA_EINVAL),
    # one state slot per (sequence, head) must fit in the fixed array
    (dict(batch=65535, hq=64, hkv=8), sa.SA_EINVAL),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert _noalloc(lib, **kw) == status
    assert lib.sink_attn_last_error().decode()


def test_decode_noalloc_limit_is_the_stated_one(lib):
    """508,398 (sequence, head) pairs fit at head_dim 64 (the header's figure); one more
    pair does not."""
    if _no_gpu():
        assert _noalloc(lib, batch=63549, hq=8, hkv=8) == sa.SA_ELAUNCH      # 508,392 pairs
    assert _noalloc(lib, batch=63550, hq=8, hkv=8) == sa.SA_EINVAL        # 508,400 pairs
    assert "state array" in lib.sink_attn_last_error().decode()
