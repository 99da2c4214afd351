"""Grouped-query attention with a learned per-head sink on MI355X (gfx950).

Thin Python binding over the C ABI of ``libsinkattn.so`` (declared in
``include/sink_attn.h``): it only checks and marshals torch tensors (device
pointers, the current HIP stream) and maps status codes to exceptions.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library has not been built the calls raise.

Operation ("GPT-OSS on day 0", Perplexity, Kernels for GPT-OSS / Sink
attention): attn = softmax(q k^T * sm_scale + sink) V with one sink logit per
query head acting as an extra softmax entry with a zero value vector.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libsinkattn.so")

SA_OK, SA_EINVAL, SA_EUNSUPPORTED, SA_ELAUNCH = 0, 1, 2, 3
SA_FP32, SA_BF16 = 0, 1
EXPORTS = ("sink_attn_prefill", "sink_attn_decode_split", "sink_attn_merge",
           "sink_attn_decode", "sink_attn_prefill_split", "sink_attn_merge_rows",
           "sink_attn_last_error", "moe_topk_softmax", "qkv_bias_rope",
           "sink_attn_prefill_state", "sink_attn_read_probe", "sink_attn_decode_noalloc")


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return os.environ.get("SINK_ATTN_LIBRARY", LIBRARY)


def load_library():
    """Load libsinkattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with gqa_attention_head_amd.build.build() "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.sink_attn_prefill.restype = ctypes.c_int
    lib.sink_attn_prefill.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      i32, i32, f32, i32, vp, vp, vp]
    lib.sink_attn_decode_split.restype = ctypes.c_int
    lib.sink_attn_decode_split.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           i32, i32, i32, f32, vp, vp, vp, vp]
    lib.sink_attn_merge.restype = ctypes.c_int
    lib.sink_attn_merge.argtypes = [ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp,
                                    vp, vp]
    lib.sink_attn_decode_noalloc.restype = ctypes.c_int
    lib.sink_attn_decode_noalloc.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                             i32, f32, vp, vp, vp]
    lib.sink_attn_decode.restype = ctypes.c_int
    lib.sink_attn_decode.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     i32, i32, f32, vp, vp, vp, vp, vp, vp]
    lib.sink_attn_prefill_split.restype = ctypes.c_int
    lib.sink_attn_prefill_split.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp]
    lib.sink_attn_merge_rows.restype = ctypes.c_int
    lib.sink_attn_merge_rows.argtypes = [ctypes.c_int, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_topk_softmax.restype = ctypes.c_int
    lib.moe_topk_softmax.argtypes = [vp, ctypes.c_int64, i32, i32, vp, vp, vp]
    lib.sink_attn_prefill_state.restype = ctypes.c_int
    lib.sink_attn_prefill_state.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, i32, f32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.qkv_bias_rope.restype = ctypes.c_int
    lib.qkv_bias_rope.argtypes = [vp, vp, vp, vp, ctypes.c_int64, i32, i32, i32, i32, vp, vp, vp,
                                  vp]
    lib.sink_attn_read_probe.restype = ctypes.c_int
    lib.sink_attn_read_probe.argtypes = [vp, ctypes.c_int64, i32, vp, vp]
    lib.sink_attn_last_error.restype = ctypes.c_char_p
    lib.sink_attn_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != SA_OK:
        msg = load_library().sink_attn_last_error().decode(errors="replace")
        raise SinkAttnError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name):
    """Raise ValueError unless tensor t (if given) has exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_qkv(q, k, v, sinks):
    """Shapes shared by every attention entry point: q [.., Hq, D], k and v
    [total_k, Hkv, D] with the same D, sinks [Hq]."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be 3-D ([rows, heads, head_dim])")
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k and v must have the same shape, got {tuple(k.shape)} and {tuple(v.shape)}")
    if q.shape[2] != k.shape[2]:
        raise ValueError(f"q and k must have the same head_dim, got {q.shape[2]} and {k.shape[2]}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"q, k and v must share one dtype, got {q.dtype}, {k.dtype}, {v.dtype}")
    if sinks.dim() != 1 or sinks.numel() != q.shape[1]:
        raise ValueError(f"sinks must be [Hq] = [{q.shape[1]}], got {tuple(sinks.shape)}")


def _check_cu(cu, name):
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError(f"{name} must be a 1-D tensor of batch + 1 >= 2 offsets")


def _check_states(parts, rows, hq, slots, d):
    pm, pd, pa = parts
    _shape(pm, (rows, hq, slots), "part_m")
    _shape(pd, (rows, hq, slots), "part_d")
    _shape(pa, (rows, hq, slots, d), "part_acc")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale,
            causal=True, out=None, lse=None, return_lse=False, stream=None):
    """Attention with sinks over a packed varlen batch; see ``sink_attn_prefill``.

    q: [total_q, Hq, D]; k, v: [total_k, Hkv, D] (bf16 or fp32, same dtype);
    sinks: [Hq] fp32; cu_seqlens_*: [B+1] int32.  Returns out (and lse [total_q, Hq]).
    """
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_q, "cu_seqlens_q")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length (batch + 1)")
    _shape(out, q.shape, "out")
    _shape(lse, q.shape[:2], "lse")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[0], q.shape[1], device=q.device, dtype=torch.float32)
    _dev(lse, "lse", torch.float32)
    _check(lib.sink_attn_prefill(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks),
                                 _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1,
                                 q.shape[1], k.shape[1], q.shape[2], int(max_seqlen_q),
                                 int(max_seqlen_k), float(sm_scale), int(bool(causal)), _ptr(out),
                                 _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse else out


def prefill_split(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  kv_chunk_size, sm_scale, causal=True, max_num_chunks=None, partials=None,
                  stream=None):
    """Split-KV prefill first pass (``sink_attn_prefill_split``): per (row, head, chunk)
    states; returns (part_m, part_d, part_acc) with rows indexing q's rows."""
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_q, "cu_seqlens_q")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length (batch + 1)")
    if max_num_chunks is None:
        max_num_chunks = max(1, -(-int(max_seqlen_k) // int(kv_chunk_size)))
    if partials is not None:
        _check_states(partials, q.shape[0], q.shape[1], int(max_num_chunks), q.shape[2])
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if partials is None:
        partials = partial_buffers(q.shape[0], q.shape[1], max_num_chunks, q.shape[2], q.device)
    pm, pd, pa = partials
    for name, t in (("part_m", pm), ("part_d", pd), ("part_acc", pa)):
        _dev(t, name, torch.float32)
    _check(lib.sink_attn_prefill_split(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, q.shape[1], k.shape[1], q.shape[2],
        int(max_seqlen_q), int(max_seqlen_k), int(kv_chunk_size), int(max_num_chunks),
        float(sm_scale), int(bool(causal)), _ptr(pm), _ptr(pd), _ptr(pa), _stream(stream)))
    return pm, pd, pa


def prefill_state(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  sm_scale, causal=True, include_sink=True, slot=0, num_slots=None,
                  partials=None, stream=None):
    """Per-row attention state over the keys of this call, into slot ``slot`` of the
    state buffers (``sink_attn_prefill_state``), for cascade attention; the buffers
    (part_m, part_d, part_acc) are [total_q, Hq, num_slots(, D)] and are returned."""
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_q, "cu_seqlens_q")
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length (batch + 1)")
    if partials is None and num_slots is None:
        raise ValueError("give num_slots or partials")
    if partials is not None:
        if partials[0].dim() != 3:
            raise ValueError("part_m must be [total_q, Hq, num_slots]")
        slots = partials[0].shape[2]
        if num_slots is not None and int(num_slots) != slots:
            raise ValueError(f"num_slots ({num_slots}) does not match the partial buffers ({slots})")
        _check_states(partials, q.shape[0], q.shape[1], slots, q.shape[2])
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if partials is None:
        partials = partial_buffers(q.shape[0], q.shape[1], num_slots, q.shape[2], q.device)
    pm, pd, pa = partials
    for name, t in (("part_m", pm), ("part_d", pd), ("part_acc", pa)):
        _dev(t, name, torch.float32)
    _check(lib.sink_attn_prefill_state(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, q.shape[1], k.shape[1], q.shape[2],
        int(max_seqlen_q), int(max_seqlen_k), float(sm_scale), int(bool(causal)),
        int(bool(include_sink)), int(slot), pm.shape[2], _ptr(pm), _ptr(pd), _ptr(pa),
        _stream(stream)))
    return pm, pd, pa


def merge_rows(part_m, part_d, part_acc, out_dtype=None, out=None, lse=None, return_lse=False,
               stream=None):
    """Log-sum-exp combination of every slot of per-row chunk states
    (``sink_attn_merge_rows``); returns out [rows, Hq, D] (and lse [rows, Hq])."""
    torch = _torch()
    if part_m.dim() != 3 or part_acc.dim() != 4:
        raise ValueError("part_m must be [rows, Hq, slots] and part_acc [rows, Hq, slots, D]")
    rows, hq, nch = part_m.shape
    d = part_acc.shape[-1]
    _check_states((part_m, part_d, part_acc), rows, hq, nch, d)
    _shape(out, (rows, hq, d), "out")
    _shape(lse, (rows, hq), "lse")
    lib = load_library()
    for name, t in (("part_m", part_m), ("part_d", part_d), ("part_acc", part_acc)):
        _dev(t, name, torch.float32)
    if out is None:
        out = torch.empty(rows, hq, d, device=part_m.device,
                          dtype=out_dtype if out_dtype is not None else torch.float32)
    _dev(out, "out")
    if lse is None and return_lse:
        lse = torch.empty(rows, hq, device=part_m.device, dtype=torch.float32)
    _dev(lse, "lse", torch.float32)
    _check(lib.sink_attn_merge_rows(_dtype_code(out), _ptr(part_m), _ptr(part_d),
                                    _ptr(part_acc), rows, hq, d, nch, _ptr(out), _ptr(lse),
                                    _stream(stream)))
    return (out, lse) if return_lse else out


def partial_buffers(batch, num_q_heads, max_num_chunks, head_dim=64, device="cuda"):
    """Allocate (part_m, part_d, part_acc) for ``decode_split``."""
    torch = _torch()
    f = dict(device=device, dtype=torch.float32)
    return (torch.empty(batch, num_q_heads, max_num_chunks, **f),
            torch.empty(batch, num_q_heads, max_num_chunks, **f),
            torch.empty(batch, num_q_heads, max_num_chunks, head_dim, **f))


def decode_split(q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, max_num_chunks,
                 sm_scale, partials=None, stream=None):
    """Split-KV decode first pass; returns (part_m, part_d, part_acc)."""
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    batch = cu_seqlens_k.numel() - 1
    if q.shape[0] != batch:
        raise ValueError("q must be [batch, Hq, D] with batch = len(cu_seqlens_k) - 1")
    if partials is not None:
        _check_states(partials, batch, q.shape[1], int(max_num_chunks), q.shape[2])
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if partials is None:
        partials = partial_buffers(batch, q.shape[1], int(max_num_chunks), q.shape[2], q.device)
    pm, pd, pa = partials
    for name, t in (("part_m", pm), ("part_d", pd), ("part_acc", pa)):
        _dev(t, name, torch.float32)
    _check(lib.sink_attn_decode_split(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks),
                                      _ptr(cu_seqlens_k), batch, q.shape[1], k.shape[1],
                                      q.shape[2], int(max_seqlen_k), int(kv_chunk_size),
                                      int(max_num_chunks), float(sm_scale), _ptr(pm), _ptr(pd),
                                      _ptr(pa), _stream(stream)))
    return pm, pd, pa


def merge(part_m, part_d, part_acc, cu_seqlens_k, kv_chunk_size, out_dtype=None, out=None,
          lse=None, return_lse=False, stream=None):
    """LSE combination of ``decode_split`` partials; returns out [B, Hq, D] (and lse)."""
    torch = _torch()
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    if part_m.dim() != 3 or part_acc.dim() != 4:
        raise ValueError("part_m must be [B, Hq, slots] and part_acc [B, Hq, slots, D]")
    batch, hq, max_num_chunks = part_m.shape
    d = part_acc.shape[-1]
    if batch != cu_seqlens_k.numel() - 1:
        raise ValueError(f"the partial buffers hold {batch} sequences, cu_seqlens_k "
                         f"{cu_seqlens_k.numel() - 1}")
    _check_states((part_m, part_d, part_acc), batch, hq, max_num_chunks, d)
    _shape(out, (batch, hq, d), "out")
    _shape(lse, (batch, hq), "lse")
    lib = load_library()
    for name, t in (("part_m", part_m), ("part_d", part_d), ("part_acc", part_acc)):
        _dev(t, name, torch.float32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if out is None:
        out = torch.empty(batch, hq, d, device=part_m.device, dtype=out_dtype or torch.bfloat16)
    _dev(out, "out")
    if lse is None and return_lse:
        lse = torch.empty(batch, hq, device=part_m.device, dtype=torch.float32)
    _dev(lse, "lse", torch.float32)
    _check(lib.sink_attn_merge(_dtype_code(out), _ptr(part_m), _ptr(part_d), _ptr(part_acc),
                               _ptr(cu_seqlens_k), int(kv_chunk_size), int(max_num_chunks), batch,
                               hq, d, _ptr(out), _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse else out


# Upper bound on the workspace the proportional-block decode is given by default.
BALANCED_WORKSPACE_BYTES = 256 << 20


def balanced_slots(batch, num_q_heads, head_dim=64, device=None):
    """State slots per (sequence, head) for ``decode(kv_chunk_size=0)``: as many as one
    sequence can be given (every block beyond one per sequence, plus two), so that no
    sequence limits the balance, within BALANCED_WORKSPACE_BYTES."""
    torch = _torch()
    cus = torch.cuda.get_device_properties(device if device is not None else 0).multi_processor_count
    ranges = cus * -(-(batch + cus // 2) // cus)
    per_slot = batch * num_q_heads * (head_dim + 2) * 4
    return int(max(2, min(ranges - batch + 2, BALANCED_WORKSPACE_BYTES // max(1, per_slot))))


class DecodeWorkspace:
    """Caller-owned scratch of ``decode``: the chunk states (m, d, acc) of the split pass."""

    def __init__(self, batch, num_q_heads, max_num_chunks, head_dim=64, device="cuda"):
        self.batch, self.num_q_heads, self.head_dim = int(batch), int(num_q_heads), int(head_dim)
        self.max_num_chunks = int(max_num_chunks)
        self.partials = partial_buffers(batch, num_q_heads, self.max_num_chunks, head_dim, device)


def decode(q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, sm_scale,
           max_num_chunks=None, workspace=None, out=None, lse=None, return_lse=False,
           stream=None):
    """Split-KV decode in one call (``sink_attn_decode``): split pass then merge, enqueued
    back to back on the stream.  kv_chunk_size > 0 cuts every sequence into chunks of that
    many keys; kv_chunk_size = 0 lets the library cut each sequence into blocks proportional
    to its length (about one workgroup per compute unit in all), using up to max_num_chunks
    state slots per sequence."""
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    batch = cu_seqlens_k.numel() - 1
    if q.shape[0] != batch:
        raise ValueError("q must be [batch, Hq, D] with batch = len(cu_seqlens_k) - 1")
    if int(kv_chunk_size) < 0:
        raise ValueError("kv_chunk_size must be >= 0")
    if workspace is not None:
        if (workspace.batch, workspace.num_q_heads, workspace.head_dim) != (batch, q.shape[1], q.shape[2]):
            raise ValueError(f"workspace is for (batch, Hq, D) = {(workspace.batch, workspace.num_q_heads, workspace.head_dim)}, "
                             f"the call has {(batch, q.shape[1], q.shape[2])}")
        if max_num_chunks is not None and int(max_num_chunks) != workspace.max_num_chunks:
            raise ValueError(f"max_num_chunks ({max_num_chunks}) differs from the workspace's "
                             f"{workspace.max_num_chunks}")
        _check_states(workspace.partials, batch, q.shape[1], workspace.max_num_chunks, q.shape[2])
    _shape(out, q.shape, "out")
    _shape(lse, (batch, q.shape[1]), "lse")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if max_num_chunks is None:
        if workspace is not None:
            max_num_chunks = workspace.max_num_chunks
        elif int(kv_chunk_size) == 0:
            max_num_chunks = balanced_slots(batch, q.shape[1], q.shape[2], q.device)
        else:
            max_num_chunks = max(1, -(-int(max_seqlen_k) // int(kv_chunk_size)))
    if workspace is None:
        workspace = DecodeWorkspace(batch, q.shape[1], max_num_chunks, q.shape[2], q.device)
    pm, pd, pa = workspace.partials
    for name, t in (("part_m", pm), ("part_d", pd), ("part_acc", pa)):
        _dev(t, name, torch.float32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if lse is None and return_lse:
        lse = torch.empty(batch, q.shape[1], device=q.device, dtype=torch.float32)
    _dev(lse, "lse", torch.float32)
    _check(lib.sink_attn_decode(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks),
                                _ptr(cu_seqlens_k), batch, q.shape[1], k.shape[1], q.shape[2],
                                int(max_seqlen_k), int(kv_chunk_size), int(max_num_chunks),
                                float(sm_scale), _ptr(pm), _ptr(pd), _ptr(pa),
                                _ptr(out), _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse else out


def decode_noalloc(q, k, v, sinks, cu_seqlens_k, max_seqlen_k, sm_scale, out=None, lse=None,
                   return_lse=False, stream=None):
    """``sink_attn_decode_noalloc``: the proportional-block decode with its states in the
    library's fixed per-device array (no workspace; the library call allocates nothing).
    Pass ``out`` (and ``lse``) to keep this call free of allocations on the torch side too."""
    torch = _torch()
    _check_qkv(q, k, v, sinks)
    _check_cu(cu_seqlens_k, "cu_seqlens_k")
    batch = cu_seqlens_k.numel() - 1
    if q.shape[0] != batch:
        raise ValueError("q must be [batch, Hq, D] with batch = len(cu_seqlens_k) - 1")
    _shape(out, q.shape, "out")
    _shape(lse, (batch, q.shape[1]), "lse")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(sinks, "sinks", torch.float32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if lse is None and return_lse:
        lse = torch.empty(batch, q.shape[1], device=q.device, dtype=torch.float32)
    _dev(lse, "lse", torch.float32)
    _check(lib.sink_attn_decode_noalloc(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks),
                                        _ptr(cu_seqlens_k), batch, q.shape[1], k.shape[1],
                                        q.shape[2], int(max_seqlen_k), float(sm_scale), _ptr(out),
                                        _ptr(lse), _stream(stream)))
    return (out, lse) if return_lse else out


def prepare_prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    sm_scale, out, causal=True, lse=None, stream=None):
    """One ``sink_attn_prefill`` call with its arguments checked and marshalled once:
    returns a function of no arguments that issues the call again (see
    ``prepare_decode``)."""
    prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sm_scale,
            causal=causal, out=out, lse=lse, stream=stream)  # checks every argument
    lib = load_library()
    args = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q),
            _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, q.shape[1], k.shape[1], q.shape[2],
            int(max_seqlen_q), int(max_seqlen_k), float(sm_scale), int(bool(causal)), _ptr(out),
            _ptr(lse), _stream(stream))
    keep = (q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, out, lse)
    fn = lib.sink_attn_prefill

    def call():
        status = fn(*args)
        if status != SA_OK:
            _check(status)
        return keep[6]

    return call


def prepare_decode(q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, sm_scale,
                   workspace, out, lse=None, stream=None):
    """One ``sink_attn_decode`` call with its arguments checked and marshalled once:
    returns a function of no arguments that issues the call again (on the stream
    current now, or ``stream``), for loops that re-run one decode over the same
    buffers.  The tensors must stay alive and keep their shapes; their contents may
    change between calls."""
    decode(q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, sm_scale,
           workspace=workspace, out=out, lse=lse, stream=stream)  # checks every argument
    lib = load_library()
    pm, pd, pa = workspace.partials
    args = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_k),
            cu_seqlens_k.numel() - 1, q.shape[1], k.shape[1], q.shape[2], int(max_seqlen_k),
            int(kv_chunk_size), workspace.max_num_chunks, float(sm_scale), _ptr(pm), _ptr(pd),
            _ptr(pa), _ptr(out), _ptr(lse), _stream(stream))
    keep = (q, k, v, sinks, cu_seqlens_k, workspace, out, lse)
    fn = lib.sink_attn_decode

    def call():
        status = fn(*args)
        if status != SA_OK:
            _check(status)
        return keep[6]

    return call


class DecodeGraph:
    """One ``decode`` call (split pass + merge) captured as a HIP graph and replayed.

    The pages' serving engine runs its decode step under graph capture; here the
    two launches of a decode call are recorded once (torch.cuda.CUDAGraph on a
    default-priority capture stream) and ``replay()`` re-runs them on the current
    stream.  Every buffer is fixed at capture: q, k, v, sinks, cu_seqlens_k, the
    workspace and the outputs.  Write new inputs into those tensors in place
    (``copy_``) before a replay; the lengths in cu_seqlens_k may change between
    replays as long as they stay within ``max_seqlen_k`` and the workspace.
    Nothing in the captured work is a memset, so replays need no re-zeroing.
    """

    def __init__(self, q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, sm_scale,
                 max_num_chunks=None, out=None, lse=None):
        torch = _torch()
        _check_qkv(q, k, v, sinks)
        _check_cu(cu_seqlens_k, "cu_seqlens_k")
        batch = cu_seqlens_k.numel() - 1
        if q.shape[0] != batch:
            raise ValueError("q must be [batch, Hq, D] with batch = len(cu_seqlens_k) - 1")
        _shape(out, q.shape, "out")
        _shape(lse, (batch, q.shape[1]), "lse")
        if max_num_chunks is None:
            max_num_chunks = (balanced_slots(batch, q.shape[1], q.shape[2], q.device)
                              if int(kv_chunk_size) == 0
                              else max(1, -(-int(max_seqlen_k) // int(kv_chunk_size))))
        self.workspace = DecodeWorkspace(batch, q.shape[1], max_num_chunks, q.shape[2], q.device)
        self.out = torch.empty_like(q) if out is None else out
        self.lse = (torch.empty(batch, q.shape[1], device=q.device, dtype=torch.float32)
                    if lse is None else lse)
        args = (q, k, v, sinks, cu_seqlens_k, max_seqlen_k, kv_chunk_size, sm_scale)
        kw = dict(max_num_chunks=max_num_chunks, workspace=self.workspace, out=self.out,
                  lse=self.lse)
        # one eager call first (argument checks, library load) on a side stream
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            decode(*args, **kw)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            decode(*args, **kw)
        self._keep = args  # the captured pointers must stay alive

    def replay(self):
        """Run the captured decode on the current stream; returns ``(out, lse)``."""
        self.graph.replay()
        return self.out, self.lse


def topk_softmax(logits, k, indices=None, weights=None, stream=None):
    """Top-K-then-softmax expert routing (``moe_topk_softmax``): logits [T, E] bf16 ->
    (indices int32 [T, k], weights bf16 [T, k]), experts in rank order."""
    torch = _torch()
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    t, e = logits.shape
    _shape(indices, (t, k), "indices")
    _shape(weights, (t, k), "weights")
    lib = load_library()
    _dev(logits, "logits", torch.bfloat16)
    if indices is None:
        indices = torch.empty(t, k, device=logits.device, dtype=torch.int32)
    if weights is None:
        weights = torch.empty(t, k, device=logits.device, dtype=torch.bfloat16)
    _dev(indices, "indices", torch.int32)
    _dev(weights, "weights", torch.bfloat16)
    if tuple(indices.shape) != (t, k) or tuple(weights.shape) != (t, k):
        raise ValueError("indices and weights must be [T, k]")
    _check(lib.moe_topk_softmax(_ptr(logits), t, e, int(k), _ptr(indices), _ptr(weights),
                                _stream(stream)))
    return indices, weights


def qkv_bias_rope(qkv, bias, positions, cos_sin, num_q_heads, num_kv_heads, q=None, k=None,
                  v=None, stream=None):
    """Pre-attention epilogue (``qkv_bias_rope``): fused projection output qkv
    [T, (Hq + 2 Hkv) * 64] bf16 plus bias, rotary embedding on the query and key heads from
    the cos/sin table [rows, 64] float32 at each token's position -> (q [T, Hq, 64],
    k [T, Hkv, 64], v [T, Hkv, 64]) bf16."""
    torch = _torch()
    d = 64
    heads = num_q_heads + 2 * num_kv_heads
    if qkv.dim() != 2 or qkv.shape[1] != heads * d:
        raise ValueError(f"qkv must be [T, {heads * d}]")
    if bias.numel() != heads * d:
        raise ValueError(f"bias must hold {heads * d} values")
    t = qkv.shape[0]
    if positions.numel() != t:
        raise ValueError("positions must be [T]")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != d:
        raise ValueError("cos_sin must be [rows, 64]")
    for name, buf, h in (("q", q, num_q_heads), ("k", k, num_kv_heads), ("v", v, num_kv_heads)):
        _shape(buf, (t, h, d), name)
    lib = load_library()
    _dev(qkv, "qkv", torch.bfloat16)
    _dev(bias, "bias", torch.bfloat16)
    _dev(positions, "positions", torch.int32)
    _dev(cos_sin, "cos_sin", torch.float32)
    outs = []
    for name, buf, h in (("q", q, num_q_heads), ("k", k, num_kv_heads), ("v", v, num_kv_heads)):
        if buf is None:
            buf = torch.empty(t, h, d, device=qkv.device, dtype=torch.bfloat16)
        _dev(buf, name, torch.bfloat16)
        if tuple(buf.shape) != (t, h, d):
            raise ValueError(f"{name} must be [T, {h}, {d}]")
        outs.append(buf)
    _check(lib.qkv_bias_rope(_ptr(qkv), _ptr(bias), _ptr(positions), _ptr(cos_sin), t,
                             num_q_heads, num_kv_heads, d, cos_sin.shape[0], _ptr(outs[0]),
                             _ptr(outs[1]), _ptr(outs[2]), _stream(stream)))
    return tuple(outs)


def read_probe(buf, num_blocks=1024, out=None, stream=None):
    """Measurement utility (``sink_attn_read_probe``): one nontemporal 16-byte-load pass
    over the bytes of the contiguous device tensor ``buf``; returns the per-workgroup XOR
    digests (uint32 values in an int32 tensor [num_blocks]), whose XOR is the XOR of every
    32-bit word of ``buf``."""
    torch = _torch()
    lib = load_library()
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(num_blocks, device=buf.device, dtype=torch.int32)
    _dev(out, "out", torch.int32)
    if out.numel() < num_blocks:
        raise ValueError("out must hold num_blocks values")
    _check(lib.sink_attn_read_probe(_ptr(buf), nbytes, int(num_blocks), _ptr(out),
                                    _stream(stream)))
    return out
