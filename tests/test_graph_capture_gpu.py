"""A whole pre-attention + attention + routing sequence captured in one HIP graph:
the QKV bias + rotary epilogue, the causal prefill on its outputs, split-KV prefill
with the row merge, and the top-K router.  Every replay, with eager work and host
synchronisation in between, equals the eager sequence bit for bit (none of these
calls allocates, synchronises or clears memory with a memset)."""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_head_amd as sa
from gqa_attention_head_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def test_captured_sequence_replays_bit_for_bit():
    hq, hkv, lens = 16, 2, [150, 64, 1]
    tokens = sum(lens)
    qkv16, _, b16, _, _, table = W.qkv_epilogue_inputs(31, tokens, hq, hkv, 64, 2048)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    qkv, bias = bf16_dev(qkv16), bf16_dev(b16)
    pos_d, tab = torch.from_numpy(pos).cuda(), torch.from_numpy(table).cuda()
    sinks = torch.from_numpy(np.random.default_rng(31).standard_normal(hq).astype(np.float32)).cuda()
    cu_d = torch.from_numpy(cu).cuda()
    logits16, _ = W.router_logits(32, 4096, 128)
    logits = bf16_dev(logits16)
    maxlen = max(lens)
    chunk = 64
    nch = -(-maxlen // chunk)
    # every output buffer allocated up front
    q = torch.empty(tokens, hq, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(tokens, hkv, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    lse = torch.empty(tokens, hq, device="cuda")
    parts = sa.partial_buffers(tokens, hq, nch, 64)
    mout = torch.empty_like(q)
    idx = torch.empty(4096, 4, device="cuda", dtype=torch.int32)
    w = torch.empty(4096, 4, device="cuda", dtype=torch.bfloat16)

    def sequence():
        sa.qkv_bias_rope(qkv, bias, pos_d, tab, hq, hkv, q=q, k=k, v=v)
        sa.prefill(q, k, v, sinks, cu_d, cu_d, maxlen, maxlen, 0.125, causal=True, out=out, lse=lse)
        sa.prefill_split(q, k, v, sinks, cu_d, cu_d, maxlen, maxlen, chunk, 0.125, causal=True,
                         max_num_chunks=nch, partials=parts)
        sa.merge_rows(*parts, out=mout)
        sa.topk_softmax(logits, 4, indices=idx, weights=w)

    sequence()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (q, k, v, out, lse, mout, idx, w)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    for t in (q, k, v, out, lse, mout, idx, w):
        t.zero_()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("q", "k", "v", "out", "lse", "merged", "idx", "w"),
                                   (q, k, v, out, lse, mout, idx, w), eager):
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), \
                f"replay {i}: {name} differs"
        _ = (torch.randn(4096, device="cuda") * 3).sum().item()  # eager work in between


def _decode_inputs(seed, batch, max_k):
    wl = W.random_case(seed, batch=batch, hq=64, hkv=8, max_k=max_k, decode=True)
    q, k, v = (bf16_dev(a) for a in wl.device_arrays())
    return (wl, q, k, v, torch.from_numpy(wl.sinks).cuda(), torch.from_numpy(wl.cu_k).cuda(),
            int(wl.seqlens_k.max()))


def _replays_equal(graph, outs, eager, scribble):
    """Replay three times, with eager work and a synchronisation in between, after
    the outputs are cleared; every replay must equal the eager result bit for bit."""
    for t in outs:
        t.zero_()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            a = got.view(torch.uint8) if got.dtype == torch.bfloat16 else got
            b = want.view(torch.uint8) if want.dtype == torch.bfloat16 else want
            assert torch.equal(a, b)
        scribble()
        torch.cuda.synchronize()


def test_captured_proportional_decode_replays_bit_for_bit():
    """DecodeGraph over the proportional-block decode (kv_chunk_size 0)."""
    wl, q, k, v, sinks, cu, max_k = _decode_inputs(41, 11, 20000)
    out = torch.empty(wl.batch, 64, 64, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(wl.batch, 64, device="cuda")
    ws = sa.DecodeWorkspace(wl.batch, 64, sa.balanced_slots(wl.batch, 64, 64))
    e_out, e_lse = sa.decode(q, k, v, sinks, cu, max_k, 0, wl.sm_scale, workspace=ws,
                             return_lse=True)
    torch.cuda.synchronize()
    g = sa.DecodeGraph(q, k, v, sinks, cu, max_k, 0, wl.sm_scale, out=out, lse=lse)
    junk = torch.empty(1 << 20, device="cuda")
    _replays_equal(g, (out, lse), (e_out, e_lse), lambda: junk.normal_())


def test_captured_noalloc_decode_replays_bit_for_bit():
    """The allocation-free decode captured in a graph: its states live in the library's
    fixed array, so the captured launches need no caller workspace at all."""
    wl, q, k, v, sinks, cu, max_k = _decode_inputs(42, 13, 30000)
    out = torch.empty(wl.batch, 64, 64, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(wl.batch, 64, device="cuda")
    sa.decode_noalloc(q, k, v, sinks, cu, max_k, wl.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sa.decode_noalloc(q, k, v, sinks, cu, max_k, wl.sm_scale, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.decode_noalloc(q, k, v, sinks, cu, max_k, wl.sm_scale, out=out, lse=lse)
    # eager work between replays that also uses the library's state array
    other = _decode_inputs(43, 5, 9000)
    _replays_equal(graph, (out, lse), eager,
                   lambda: sa.decode_noalloc(*other[1:6], other[6], other[0].sm_scale))
