#!/usr/bin/env python3
"""Benchmark of grouped-query attention with per-head sinks on one MI355X.

One step = one split-KV decode call (split pass, then the log-sum-exp merge,
enqueued back to back on the stream) of the batched gpt-oss-shaped decode
workload: 32 sequences x 1 query token over 4096 cached keys, 64 query heads on
8 KV heads, head_dim 64, bf16, 8 KV chunks of 512 keys per sequence.  `value` is
the K/V bytes that step reads (268,435,456 B) divided by the step's GPU time, in
GB/s: the timed steps are bracketed by a synchronisation on both sides, and an
event pair on the launch stream around their back-to-back launches gives the GPU
time (the host clock's figure for the same bracket is `wall_ms_per_step`).  Each
step is a call prepared once (arguments checked and marshalled), the warm-up runs
at least 100 steps and 200 ms, inputs are resident in HBM before timing starts,
and the steps rotate over several copies of K/V (>= 1 GiB in total) so the
256 MB last-level cache cannot serve repeats.

The same JSON line carries the prefill half of the metric (causal prefill,
4 x 4096 tokens, 64/8 heads, bf16) as achieved TFLOP/s over the causal pairs,
the roofline of the dominant kernel (timed with HIP events on the stream it
runs on), the other workloads (tiny fp32 prefill, long-context ragged decode,
mixed packed batch with each part against its own roofline) and the fp64 CPU
oracle timed on the host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode KV GB/s (% HBM peak); prefill TFLOP/s (% bf16 MFMA peak)"
KV_COPIES = 5                  # 5 x 268 MB rotated


def warm_up(fn, launches: int, min_ms: float = 0.0):
    """Untimed launches: at least `launches`, and more until `min_ms` of wall time has
    passed (the clocks settle over some tens of milliseconds after the load changes)."""
    t0 = time.perf_counter()
    i = 0
    while i < launches or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn(i)
        i += 1
        if i % 20 == 0:
            _sync()
    _sync()
    return i


def _sync():
    import torch
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_decode(steps: int, warmup: int):
    """The headline step: one sink_attn_decode call (split pass + merge) on the batched
    decode workload, each call prepared once (arguments checked and marshalled) so the
    host issues steps faster than the GPU runs them."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    wl = W.batched_decode()
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    q = up(wl.q16)
    k0, v0 = up(wl.k16), up(wl.v16)
    ks = [k0] + [k0.clone() for _ in range(KV_COPIES - 1)]
    vs = [v0] + [v0.clone() for _ in range(KV_COPIES - 1)]
    sinks = torch.from_numpy(wl.sinks).to(dev)
    cu_k = torch.from_numpy(wl.cu_k).to(dev)
    max_lk = int(wl.seqlens_k.max())
    chunk = wl.kv_chunk
    nch = -(-max_lk // chunk)
    ws = sa.DecodeWorkspace(wl.batch, wl.num_q_heads, nch, wl.head_dim, dev)
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim, device=dev, dtype=torch.bfloat16)
    lse = torch.empty(wl.batch, wl.num_q_heads, device=dev, dtype=torch.float32)
    calls = [sa.prepare_decode(q, ks[j], vs[j], sinks, cu_k, max_lk, chunk, wl.sm_scale, ws, out,
                               lse) for j in range(KV_COPIES)]

    def step(i):
        calls[i % KV_COPIES]()

    # The clocks need some tens of milliseconds of load to settle after idle or a
    # change of load: at least 100 steps and 200 ms of warm-up.
    warm_up(step, max(warmup, 100), 200.0)
    # The timed steps, bracketed by a synchronisation on both sides; their GPU time
    # comes from an event pair on the launch stream around the back-to-back launches,
    # the host clock gives the wall time of the same bracket.
    e0, e1 = _events()
    _sync()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    _sync()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms_per_step = e0.elapsed_time(e1) / steps
    # Average launch duration of the step's dominant kernel (the split pass), with
    # events on the stream it runs on, over a run of back-to-back launches.
    split_steps = max(steps, 200)
    warm_up(lambda i: sa.decode_split(q, ks[i % KV_COPIES], vs[i % KV_COPIES], sinks, cu_k, max_lk,
                                      chunk, nch, wl.sm_scale, partials=ws.partials), 50, 60.0)
    e0.record()
    for i in range(split_steps):
        j = i % KV_COPIES
        sa.decode_split(q, ks[j], vs[j], sinks, cu_k, max_lk, chunk, nch, wl.sm_scale,
                        partials=ws.partials)
    e1.record()
    _sync()
    split_ms = e0.elapsed_time(e1) / split_steps
    # The same step replayed from captured HIP graphs (one per K/V copy).
    graphs = [sa.DecodeGraph(q, ks[j], vs[j], sinks, cu_k, max_lk, chunk, wl.sm_scale, out=out,
                             lse=lse) for j in range(KV_COPIES)]
    warm_up(lambda i: graphs[i % KV_COPIES].replay(), max(warmup, 100), 200.0)
    e0.record()
    for i in range(steps):
        graphs[i % KV_COPIES].replay()
    e1.record()
    _sync()
    graph_ms = e0.elapsed_time(e1) / steps
    # one step at a time, the host waiting for each (a serving loop that needs the
    # result before the next step): eager launches against the captured graph
    sync_ms = {}
    for name, fn in (("eager", step), ("graph", lambda i: graphs[i % KV_COPIES].replay())):
        for i in range(10):
            fn(i)
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
            torch.cuda.synchronize()
        sync_ms[name] = (time.perf_counter() - t0) * 1e3 / steps
    # distribution of single steps (an event pair around each step adds its own gap)
    warm_up(step, 100, 100.0)
    evs = [_events() for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    _sync()
    step_ms = np.array([a.elapsed_time(b) for a, b in evs])
    kv_bytes = wl.kv_bytes()
    return dict(
        workload=wl.name, kv_bytes=kv_bytes, ms_per_step=ms_per_step, wall_ms_per_step=wall_ms,
        gbs=kv_bytes / (ms_per_step * 1e-3) / 1e9,
        split_ms_mean=float(split_ms), graph_ms_per_step=graph_ms, sync_ms=sync_ms,
        step_ms_p10_p50_p90=[float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        batch=wl.batch, kv_len=int(max_lk), chunk=chunk, num_chunks=nch, wl=wl)


def bench_tiny_prefill(steps: int = 400):
    """The tiny fp32 causal prefill (1 x 128 tokens, 4 query heads on 1 KV head), timed two
    ways: back-to-back calls (GPU time per call, from an event pair) and one call at a time
    with the host waiting for each.  The fp32 kernel gives four lanes to each (row, head)
    pair, so this size runs 32 workgroups of 64 lanes, each walking up to four 32-key
    tiles one after another (the next tile's loads in flight while one is used): the call
    is bound by that short chain, not by the launch."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    wl = W.tiny_prefill_fp32()
    dev = torch.device("cuda", 0)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (wl.q32, wl.k32, wl.v32))
    sinks = torch.from_numpy(wl.sinks).to(dev)
    cu_q, cu_k = torch.from_numpy(wl.cu_q).to(dev), torch.from_numpy(wl.cu_k).to(dev)
    out = torch.empty_like(q)
    lq = int(wl.seqlens_q.max())
    call = sa.prepare_prefill(q, k, v, sinks, cu_q, cu_k, lq, lq, wl.sm_scale, out, causal=True)
    warm_up(lambda i: call(), 100, 60.0)
    e0, e1 = _events()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    _sync()
    gpu_ms = e0.elapsed_time(e1) / steps
    for _ in range(20):
        call()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
        torch.cuda.synchronize()
    synced_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"workload": "tiny_prefill_fp32_b1_s128_hq4_hkv1_d64", "dtype": "f32",
            "ms_back_to_back": round(gpu_ms, 5), "ms_host_synced": round(synced_ms, 5),
            "flops": wl.prefill_flops(),
            "note": "fp32 vector-ALU kernel, 32 workgroups at this size (four lanes per row and head): time only; parity is checked in the CPU baseline leg and the tests",
            "_out": out.cpu().numpy(), "_wl": wl}


def bench_prefill(steps: int, warmup: int):
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    wl = W.causal_prefill()
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(wl.q16), up(wl.k16), up(wl.v16)
    sinks = torch.from_numpy(wl.sinks).to(dev)
    cu_q = torch.from_numpy(wl.cu_q).to(dev)
    cu_k = torch.from_numpy(wl.cu_k).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], device=dev, dtype=torch.float32)
    lq = int(wl.seqlens_q.max())

    def step():
        sa.prefill(q, k, v, sinks, cu_q, cu_k, lq, lq, wl.sm_scale, causal=True, out=out, lse=lse)

    # The clocks need some tens of milliseconds of load to settle after idle or a
    # change of load: at least 50 launches and 60 ms of warm-up before the timed run.
    warm_up(lambda i: step(), max(warmup, 50), 60.0)
    # back-to-back launches between one event pair on the launch stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    _sync()
    mean_ms = ev[0].elapsed_time(ev[1]) / steps
    # distribution of single launches (an event pair around each)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        step()
        evs[i][1].record()
    _sync()
    one = np.array([e[0].elapsed_time(e[1]) for e in evs])
    flops = wl.prefill_flops()
    return dict(workload=wl.name, flops=flops, ms_mean=mean_ms,
                ms_p10_p50_p90=[float(np.percentile(one, q)) for q in (10, 50, 90)],
                tflops=flops / (mean_ms * 1e-3) / 1e12, wl=wl, gemm_tflops=library_gemm_tflops())


def read_ceiling(copies: int = 5, nbytes: int = 268435456, steps: int = 50):
    """The device's practical streaming-read rate: the library's read yardstick
    (nontemporal 16-byte loads, the decode's K/V access) over `copies` rotated buffers
    of the decode's K/V size, so the last-level cache cannot serve repeats."""
    import torch
    import gqa_attention_head_amd as sa
    bufs = [torch.ones(nbytes // 4, device="cuda", dtype=torch.int32) for _ in range(copies)]
    out = torch.empty(1024, device="cuda", dtype=torch.int32)
    warm_up(lambda i: sa.read_probe(bufs[i % copies], 1024, out), 50, 60.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(steps):
        sa.read_probe(bufs[i % copies], 1024, out)
    ev[1].record()
    _sync()
    del bufs
    return round(nbytes / (ev[0].elapsed_time(ev[1]) / steps * 1e-3) / 1e9, 1)


def context_hbm():
    """Context for the HBM roofline: the library's streaming-read yardstick, and what
    torch's own kernels sustain on this GPU, a reduction (reads 2 GiB) and a copy (reads
    and writes 1 GiB)."""
    import torch
    res = {"read_probe_gbs": read_ceiling()}
    x = torch.ones(1 << 30, device="cuda", dtype=torch.bfloat16)
    y = torch.empty(1 << 29, device="cuda", dtype=torch.bfloat16)
    for name, fn, nbytes in (("sum_read_gbs", lambda: x.sum(dtype=torch.float32), 2 << 30),
                             ("copy_gbs", lambda: y.copy_(x[: 1 << 29]), 2 << 30)):
        for _ in range(5):
            fn()
        _sync()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(20):
            fn()
        ev[1].record()
        _sync()
        res[name] = round(nbytes / (ev[0].elapsed_time(ev[1]) / 20 * 1e-3) / 1e9, 1)
    del x, y
    return res


def library_gemm_tflops(n: int = 8192, steps: int = 50, warmup: int = 20) -> float:
    """Context for the MFMA roofline: what the vendor GEMM (torch.matmul -> hipBLASLt)
    sustains on a square bf16 n x n x n product on this GPU, right after the prefill."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(warmup):
        torch.matmul(a, b, out=c)
    _sync()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        torch.matmul(a, b, out=c)
    ev[1].record()
    _sync()
    ms = ev[0].elapsed_time(ev[1]) / steps
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def bench_prefill_groups(groups=(1, 2, 4, 16), steps: int = 50):
    """The causal prefill shape (4 x 4096, 64 query heads) with other group sizes
    (Hkv = 64 / G): TFLOP/s per G, as context for the G = 8 line."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    dev = torch.device("cuda", 0)
    res = {}
    for g in groups:
        wl = W.make_workload(f"prefill_bf16_b4_s4096_h64g{g}_d64", dtype="bf16", kind="prefill",
                             seqlens_q=[4096] * 4, seqlens_k=[4096] * 4, num_q_heads=64,
                             num_kv_heads=64 // g, head_dim=64, seed=3, causal=True)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        q, k, v = up(wl.q16), up(wl.k16), up(wl.v16)
        sinks = torch.from_numpy(wl.sinks).to(dev)
        cu = torch.from_numpy(wl.cu_q).to(dev)
        out = torch.empty_like(q)
        step = lambda i: sa.prefill(q, k, v, sinks, cu, cu, 4096, 4096, wl.sm_scale, causal=True, out=out)
        warm_up(step, 20, 30.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for i in range(steps):
            step(i)
        ev[1].record()
        _sync()
        ms = ev[0].elapsed_time(ev[1]) / steps
        res[f"G{g}"] = {"ms": round(ms, 4), "tflops": round(wl.prefill_flops() / (ms * 1e-3) / 1e12, 1)}
    return res


LONG_KV = dict(lq=256, lk=131072, chunk=16384)  # chunked prefill over a long cache


def bench_prefill_long_kv(steps: int, warmup: int):
    """A chunked prefill (256 new tokens over 131072 cached keys, 64/8 heads, bf16):
    the unsplit kernel (64 workgroups) against the split-KV pass + row merge."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    lq, lk, chunk = LONG_KV["lq"], LONG_KV["lk"], LONG_KV["chunk"]
    wl = W.make_workload(f"chunked_prefill_bf16_q{lq}_kv{lk}_h64g8_d64", dtype="bf16",
                         kind="prefill", seqlens_q=[lq], seqlens_k=[lk], num_q_heads=64,
                         num_kv_heads=8, head_dim=64, seed=11, causal=True)
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(wl.q16), up(wl.k16), up(wl.v16)
    sinks = torch.from_numpy(wl.sinks).to(dev)
    cu_q = torch.from_numpy(wl.cu_q).to(dev)
    cu_k = torch.from_numpy(wl.cu_k).to(dev)
    nch = -(-lk // chunk)
    parts = sa.partial_buffers(lq, 64, nch, 64, dev)
    out = torch.empty_like(q)

    def unsplit():
        sa.prefill(q, k, v, sinks, cu_q, cu_k, lq, lk, wl.sm_scale, causal=True, out=out)

    def split():
        sa.prefill_split(q, k, v, sinks, cu_q, cu_k, lq, lk, chunk, wl.sm_scale,
                         max_num_chunks=nch, partials=parts)
        sa.merge_rows(*parts, out=out)

    res = {}
    for name, fn in (("unsplit", unsplit), ("split", split)):
        for _ in range(warmup):
            fn()
        _sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        _sync()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms": round(ms, 4), "tflops": round(wl.prefill_flops() / (ms * 1e-3) / 1e12, 2)}
    res["split"]["kv_chunk"] = chunk
    return dict(workload=wl.name, flops=wl.prefill_flops(), **res)


def _time_ms(fn, steps: int, warmup: int) -> float:
    import torch
    warm_up(lambda i: fn(), warmup, 60.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    _sync()
    return e0.elapsed_time(e1) / steps


def _time_calls(calls, steps: int, warmup: int, min_ms: float = 60.0) -> float:
    """Mean GPU time of one call, from an event pair around `steps` back-to-back calls
    that rotate over `calls`, after a warm-up of at least `warmup` calls and `min_ms`."""
    n = len(calls)
    warm_up(lambda i: calls[i % n](), warmup, min_ms)
    e0, e1 = _events()
    e0.record()
    for i in range(steps):
        calls[i % n]()
    e1.record()
    _sync()
    return e0.elapsed_time(e1) / steps


def bench_ragged_decode(steps: int = 40, warmup: int = 20):
    """The long-context ragged decode (8 sequences, KV lengths of the seeded workload, 1024 to
    131072 keys, 64/8 heads, bf16): one decode call (split pass + merge) per step, with the
    configured 2048-key chunks and with proportional blocks (kv_chunk_size 0: one
    workgroup per compute unit).  K/V (1.6 GB, above the last-level cache) are drawn on the
    device from a seeded generator: the values do not change the timing, the lengths do."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    lens = W.ragged_decode_lengths()
    chunk, hq, hkv, d = 2048, 64, 8, 64
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    total = int(lens.sum())
    k = torch.randn(total, hkv, d, device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn(total, hkv, d, device=dev, generator=g).to(torch.bfloat16)
    q = torch.randn(len(lens), hq, d, device=dev, generator=g).to(torch.bfloat16)
    sinks = 2.0 * torch.randn(hq, device=dev, generator=g)
    cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    max_k = int(lens.max())
    out = torch.empty_like(q)
    kv_bytes = total * hkv * d * 2 * 2
    res = {"workload": f"ragged_decode_bf16_b{len(lens)}_kv1024-131072_h64g8_d64",
           "kv_lengths": [int(x) for x in lens], "kv_bytes": kv_bytes}
    for name, c, slots in (("fixed_chunk_2048", chunk, -(-max_k // chunk)),
                           ("proportional_blocks", 0, sa.balanced_slots(len(lens), hq, d, dev))):
        ws = sa.DecodeWorkspace(len(lens), hq, slots, d, dev)
        ms = _time_calls([sa.prepare_decode(q, k, v, sinks, cu_k, max_k, c, 0.125, ws, out)],
                         steps, warmup)
        gbs = kv_bytes / (ms * 1e-3) / 1e9
        res[name] = {"kv_chunk_size": c, "slots": slots, "ms": round(ms, 4),
                     "value": round(gbs, 2), "unit": "GB/s", "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    best = res["proportional_blocks"]
    res.update(ms=best["ms"], value=best["value"], unit="GB/s", hbm_frac=best["hbm_frac"],
               mode="proportional_blocks")
    del k, v
    return res


MIXED_COPIES = 4  # rotated copies of the mixed batch's K/V (4 x 332 MB)


def bench_mixed_varlen(steps: int = 40, warmup: int = 20, side=None):
    """The mixed packed batch (4 prefill chunks of 512-2048 new tokens over 0-8192 cached
    keys, then 12 single-token decodes over 1024-32768 keys, 64/8 heads, bf16).  Each part
    against its own roofline: the prefill chunks in one prefill call (TFLOP/s over their
    causal pairs, against 2.5 PF) and the 12 decodes in one decode call (K/V GB/s, against
    8 TB/s; proportional blocks, and 2048-key chunks for reference).  Then the whole batch:
    one prefill call over all 16 sequences, the two calls on one stream, and the two calls
    on two streams, each against max(prefill flops / 2.5 PF, decode bytes / 8 TB/s).  The
    timed calls rotate over 4 copies of K/V (1.3 GB) so that the last-level cache cannot
    serve repeats."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    wl = W.mixed_varlen()
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    q = up(wl.q16)
    k0, v0 = up(wl.k16), up(wl.v16)
    ks = [k0] + [k0.clone() for _ in range(MIXED_COPIES - 1)]
    vs = [v0] + [v0.clone() for _ in range(MIXED_COPIES - 1)]
    sinks = torch.from_numpy(wl.sinks).to(dev)
    cu_q = torch.from_numpy(wl.cu_q).to(dev)
    cu_k = torch.from_numpy(wl.cu_k).to(dev)
    lq, lk = wl.seqlens_q, wl.seqlens_k
    npre = int((lq > 1).sum())
    assert (lq[:npre] > 1).all() and (lq[npre:] == 1).all(), "prefill chunks come first"
    out = torch.empty_like(q)
    flops_pre = sum(4 * 64 * 64 * (int(a) * (int(b) - int(a)) + int(a) * (int(a) + 1) // 2)
                    for a, b in zip(lq[:npre], lk[:npre]))
    bytes_dec = int(lk[npre:].sum()) * 8 * 64 * 2 * 2
    r0 = int(wl.cu_q[npre])
    ndec = len(lq) - npre
    q_dec, out_dec = q[r0:], out[r0:]
    cu_pre, cu_kpre, cu_dec = cu_q[:npre + 1], cu_k[:npre + 1], cu_k[npre:]
    max_q_pre, max_k_pre = int(lq[:npre].max()), int(lk[:npre].max())
    max_k_dec = int(lk[npre:].max())
    ws_fixed = sa.DecodeWorkspace(ndec, 64, -(-max_k_dec // 2048), 64, dev)
    ws_prop = sa.DecodeWorkspace(ndec, 64, sa.balanced_slots(ndec, 64, 64, dev), 64, dev)
    pre = [sa.prepare_prefill(q, ks[j], vs[j], sinks, cu_pre, cu_kpre, max_q_pre, max_k_pre,
                              wl.sm_scale, out) for j in range(MIXED_COPIES)]
    dec = [sa.prepare_decode(q_dec, ks[j], vs[j], sinks, cu_dec, max_k_dec, 0, wl.sm_scale,
                             ws_prop, out_dec) for j in range(MIXED_COPIES)]
    dec_fixed = [sa.prepare_decode(q_dec, ks[j], vs[j], sinks, cu_dec, max_k_dec, 2048,
                                   wl.sm_scale, ws_fixed, out_dec) for j in range(MIXED_COPIES)]
    one = [sa.prepare_prefill(q, ks[j], vs[j], sinks, cu_q, cu_k, int(lq.max()), int(lk.max()),
                              wl.sm_scale, out) for j in range(MIXED_COPIES)]
    if side is None:
        side = torch.cuda.Stream(device=dev)  # default priority
    side_dec = []
    with torch.cuda.stream(side):
        side_dec = [sa.prepare_decode(q_dec, ks[j], vs[j], sinks, cu_dec, max_k_dec, 0,
                                      wl.sm_scale, ws_prop, out_dec) for j in range(MIXED_COPIES)]
    torch.cuda.synchronize()

    def two_calls(j):
        return lambda: (pre[j](), dec[j]())

    def two_streams(j):
        # the MFMA-bound prefill and the HBM-bound decode overlap on two streams
        def run():
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            side_dec[j]()
            pre[j]()
            main.wait_stream(side)
        return run

    roof_ms = max(flops_pre / (BF16_PEAK_TFLOPS * 1e12), bytes_dec / (HBM_PEAK_GBS * 1e9)) * 1e3
    res = {"workload": wl.name, "prefill_flops": flops_pre, "decode_kv_bytes": bytes_dec,
           "kv_copies_rotated": MIXED_COPIES, "roofline_ms": round(roof_ms, 4)}
    ms = _time_calls(pre, steps, warmup)
    tf = flops_pre / (ms * 1e-3) / 1e12
    res["prefill_part"] = {"ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
                           "roofline": {"bound": "mfma", "peak": BF16_PEAK_TFLOPS,
                                        "frac": round(tf / BF16_PEAK_TFLOPS, 4)}}
    for name, calls in (("decode_part", dec), ("decode_part_fixed_chunk_2048", dec_fixed)):
        ms = _time_calls(calls, steps, warmup)
        gbs = bytes_dec / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "value": round(gbs, 2), "unit": "GB/s",
                     "roofline": {"bound": "hbm", "peak": HBM_PEAK_GBS,
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    res["decode_part"]["mode"] = "proportional_blocks"
    for name, calls in (("one_prefill_call", one),
                        ("prefill_plus_decode_calls", [two_calls(j) for j in range(MIXED_COPIES)]),
                        ("prefill_and_decode_on_two_streams",
                         [two_streams(j) for j in range(MIXED_COPIES)])):
        ms = _time_calls(calls, steps, warmup)
        res[name] = {"ms": round(ms, 4), "roofline_frac": round(roof_ms / ms, 4)}
    del ks, vs
    return res


ROUTER = dict(tokens=1 << 20, experts=128, k=4, copies=2)


def bench_router(steps: int, warmup: int):
    """Top-K-then-softmax expert routing over 2^20 tokens x 128 experts, top-4 (bf16
    logits, two rotated copies of 268 MB so the last-level cache cannot serve repeats)."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    t, e, k = ROUTER["tokens"], ROUTER["experts"], ROUTER["k"]
    bits, _ = W.router_logits(12, t, e)
    dev = torch.device("cuda", 0)
    lg0 = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    lgs = [lg0] + [lg0.clone() for _ in range(ROUTER["copies"] - 1)]
    idx = torch.empty(t, k, device=dev, dtype=torch.int32)
    w = torch.empty(t, k, device=dev, dtype=torch.bfloat16)
    warm_up(lambda i: sa.topk_softmax(lgs[i % len(lgs)], k, indices=idx, weights=w), warmup, 60.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        sa.topk_softmax(lgs[i % len(lgs)], k, indices=idx, weights=w)
    e1.record()
    _sync()
    ms = e0.elapsed_time(e1) / steps
    nbytes = t * e * 2 + t * k * (4 + 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"router_topk_softmax_bf16_t{t}_e{e}_k{k}", "ms": round(ms, 5),
            "roofline": {"kernel": f"topk_softmax_kernel<{e}, {k}>", "bound": "hbm",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}}


EPILOGUE = dict(tokens=16384, hq=64, hkv=8, max_pos=8192, copies=2)


def bench_epilogue(steps: int, warmup: int):
    """QKV bias + rotary epilogue over 16384 tokens x (64 + 2 x 8) heads of 64 (bf16,
    two rotated copies of the 168 MB projection output)."""
    import torch
    import gqa_attention_head_amd as sa
    from gqa_attention_head_amd import workloads as W

    t, hq, hkv = EPILOGUE["tokens"], EPILOGUE["hq"], EPILOGUE["hkv"]
    qkv16, _, b16, _, pos, table = W.qkv_epilogue_inputs(13, t, hq, hkv, 64, EPILOGUE["max_pos"])
    dev = torch.device("cuda", 0)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    x0 = bf(qkv16)
    xs = [x0] + [x0.clone() for _ in range(EPILOGUE["copies"] - 1)]
    bias, pos_d, tab = bf(b16), torch.from_numpy(pos).to(dev), torch.from_numpy(table).to(dev)
    q = torch.empty(t, hq, 64, device=dev, dtype=torch.bfloat16)
    k = torch.empty(t, hkv, 64, device=dev, dtype=torch.bfloat16)
    v = torch.empty(t, hkv, 64, device=dev, dtype=torch.bfloat16)
    call = lambda i: sa.qkv_bias_rope(xs[i % len(xs)], bias, pos_d, tab, hq, hkv, q=q, k=k, v=v)
    warm_up(call, warmup, 60.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    _sync()
    ms = e0.elapsed_time(e1) / steps
    heads = hq + 2 * hkv
    # projection output read + q/k/v written + bias + positions + the table rows used
    nbytes = 2 * t * heads * 64 * 2 + heads * 64 * 2 + t * 4 + len(np.unique(pos)) * 64 * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"qkv_bias_rope_bf16_t{t}_hq{hq}_hkv{hkv}_d64", "ms": round(ms, 5),
            "roofline": {"kernel": "qkv_rope_kernel", "bound": "hbm", "achieved": round(gbs, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": int(nbytes)}}


def _cpu_threads():
    """Threads for the oracle: the cores this process may run on (its affinity set),
    capped by OMP_NUM_THREADS when that is set (the GPU machine sets it to its CPU share)."""
    n = _affinity()
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(omp)) if omp.isdigit() and int(omp) > 0 else n


def _affinity():
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def _median_rate(run, units: float, rounds: int = 3, min_s: float = 2.0):
    """Median over `rounds` timing rounds (each repeating `run` for at least `min_s`) of
    units per second; returns (rate, seconds per run, runs per round)."""
    rates, per_run, reps = [], [], []
    for _ in range(rounds):
        t0 = time.perf_counter()
        n = 0
        while True:
            run()
            n += 1
            if time.perf_counter() - t0 >= min_s:
                break
        sec = (time.perf_counter() - t0) / n
        rates.append(units / sec)
        per_run.append(sec)
        reps.append(n)
    i = int(np.argsort(rates)[len(rates) // 2])
    return rates[i], per_run[i], reps[i]


def cpu_baseline(dec_wl, pre_wl, tiny=None):
    """The fp64 oracle, untuned, on the host: decode over whole sequences of the decode
    workload, prefill over sampled query rows of the prefill workload, each the median of
    three timing rounds; and the tiny fp32 prefill's GPU output checked against it."""
    import oracle
    orc = oracle.default()
    threads = _cpu_threads()
    # decode: the first 8 of 32 sequences (all 64 heads, all 4096 keys each)
    nseq = 8
    sub_rows = np.arange(nseq, dtype=np.int64)
    dec_bytes = int(dec_wl.seqlens_k[:nseq].sum()) * dec_wl.num_kv_heads * dec_wl.head_dim * 2 * 2
    dec_rate, dec_s, reps = _median_rate(
        lambda: orc.workload(dec_wl, rows=sub_rows, nthreads=threads), dec_bytes, min_s=3.0)
    # prefill: 16 rows from the end of each sequence (the longest rows), all heads
    rows = np.concatenate([np.arange(int(pre_wl.cu_q[b + 1]) - 16, int(pre_wl.cu_q[b + 1]))
                           for b in range(pre_wl.batch)]).astype(np.int64)
    pairs = 0
    for r in rows:
        b = int(np.searchsorted(pre_wl.cu_q, r, side="right") - 1)
        i = int(r - pre_wl.cu_q[b])
        pairs += int(pre_wl.seqlens_k[b]) - int(pre_wl.seqlens_q[b]) + i + 1
    pre_flops = 4 * pre_wl.head_dim * pre_wl.num_q_heads * pairs
    pre_rate, pre_s, pre_reps = _median_rate(
        lambda: orc.workload(pre_wl, rows=rows, nthreads=threads), pre_flops, min_s=2.0)
    # decode on one thread: the first sequence
    dec1_bytes = int(dec_wl.seqlens_k[0]) * dec_wl.num_kv_heads * dec_wl.head_dim * 2 * 2
    dec1_rate, dec1_s, dec1_reps = _median_rate(
        lambda: orc.workload(dec_wl, rows=np.arange(1, dtype=np.int64), nthreads=1), dec1_bytes,
        min_s=1.0)
    res = dict(
        value=dec_rate / 1e9, unit="GB/s", cores=threads, kind="oracle",
        sample=f"decode: {nseq} of {dec_wl.batch} sequences x 64 heads x 4096 keys "
               f"({dec_bytes} B of K/V), median of 3 rounds of {reps} run(s), {dec_s:.3f} s each",
        cores_note=f"{threads} threads: this process's CPU set ({_affinity()} cores) capped by "
                   f"OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')}; "
                   f"os.cpu_count() = {os.cpu_count()}",
        cpu_model=_cpu_model(),
        decode_one_thread=dict(value=dec1_rate / 1e9, unit="GB/s", cores=1,
                               sample=f"decode: 1 sequence x 64 heads x 4096 keys, median of 3 "
                                      f"rounds of {dec1_reps} run(s), {dec1_s:.3f} s each"),
        prefill=dict(value=pre_rate / 1e12, unit="TFLOP/s", cores=threads,
                     sample=f"prefill: {rows.size} query rows (last 16 of each sequence) x 64 "
                            f"heads, median of 3 rounds of {pre_reps} run(s), {pre_s:.3f} s each"),
        router=_cpu_router(), qkv_epilogue=_cpu_epilogue())
    if tiny is not None:
        wl = tiny["_wl"]
        t0 = time.perf_counter()
        ref, _ = orc.workload(wl, nthreads=threads)
        sec = time.perf_counter() - t0
        err = float(np.abs(tiny["_out"].astype(np.float64) - ref).max())
        res["tiny_prefill_fp32"] = dict(seconds=round(sec, 5), gpu_max_abs_err=err,
                                        tolerance=1e-5, within_tolerance=bool(err <= 1e-5))
    return res


def _cpu_model() -> str:
    """The host CPU as the kernel names it: lscpu's vendor, model name, family/model/stepping
    and sockets, else /proc/cpuinfo's model name."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        f = {}
        for line in out.splitlines():
            if ":" in line:
                key, val = line.split(":", 1)
                f.setdefault(key.strip(), val.strip())
        if f.get("Model name"):
            fam = "/".join(f.get(k, "?") for k in ("CPU family", "Model", "Stepping"))
            return (f"{f.get('Vendor ID', '')} {f['Model name']} (family/model/stepping {fam}, "
                    f"{f.get('Socket(s)', '?')} socket(s), {f.get('CPU(s)', '?')} logical CPUs)").strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_router():
    """The router oracle (numpy, fp64) on the first 65536 tokens of the router workload."""
    from oracle.router import topk_softmax as ref
    from gqa_attention_head_amd import workloads as W
    t, e, k = 1 << 16, ROUTER["experts"], ROUTER["k"]
    _, vals = W.router_logits(12, t, e)
    t0 = time.perf_counter()
    ref(vals, k)
    sec = time.perf_counter() - t0
    nbytes = t * e * 2 + t * k * 6
    return dict(value=nbytes / sec / 1e9, unit="GB/s",
                sample=f"router: {t} tokens x {e} experts, top-{k}, {sec:.3f} s")


def _cpu_epilogue():
    """The epilogue oracle (numpy, fp64) on 1024 tokens of the epilogue workload."""
    from oracle.rope import qkv_bias_rope as ref
    from gqa_attention_head_amd import workloads as W
    t, hq, hkv = 1024, EPILOGUE["hq"], EPILOGUE["hkv"]
    _, qkv32, _, b32, pos, table = W.qkv_epilogue_inputs(13, t, hq, hkv, 64, EPILOGUE["max_pos"])
    t0 = time.perf_counter()
    ref(qkv32, b32, pos, table, hq, hkv, 64)
    sec = time.perf_counter() - t0
    nbytes = 2 * t * (hq + 2 * hkv) * 64 * 2
    return dict(value=nbytes / sec / 1e9, unit="GB/s",
                sample=f"epilogue: {t} tokens x {hq + 2 * hkv} heads, {sec:.3f} s")


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_decode_b32_kv4096_prefill_b4_s4096.md")
TRAFFIC_SOURCES = {
    "decode": ("gqa_attention_head_amd/csrc/common.h", "gqa_attention_head_amd/csrc/decode_tile.h",
               "gqa_attention_head_amd/csrc/decode.hip"),
    "prefill": ("gqa_attention_head_amd/csrc/common.h", "gqa_attention_head_amd/csrc/decode_tile.h",
                "gqa_attention_head_amd/csrc/prefill.hip"),
    "router": ("gqa_attention_head_amd/csrc/common.h", "gqa_attention_head_amd/csrc/router.hip"),
    "epilogue": ("gqa_attention_head_amd/csrc/common.h", "gqa_attention_head_amd/csrc/epilogue.hip"),
}


def measured_traffic():
    """Calibrated HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None for a kernel whose sources changed since those counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return {}
    out = {}
    for key, files in TRAFFIC_SOURCES.items():
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read()
                                    for f in files)).hexdigest()
        m = re.search(rf"traffic_{key}_source_sha256: ([0-9a-f]+)", text)
        v = re.search(rf"traffic_{key}_bytes_per_launch: (\d+)", text)
        if m and v and m.group(1) == h:
            out[key] = int(v.group(1))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode only (skips the prefill, long-KV prefill, router and epilogue legs)")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this attention path has no multi-GPU leg.", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    # HIP binds a stream to one of the process's hardware queues (GPU_MAX_HW_QUEUES,
    # 4 by default) round-robin when the stream first submits work, and kernels on
    # one hardware queue run in order.  The mixed batch's second stream therefore gets
    # its first work here, right after the default stream's, so that the two land on
    # different queues whatever the later legs create (a side stream first used after
    # the decode section's graph-capture streams shared the default stream's queue).
    torch.zeros(1, device="cuda").add_(1)
    side = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(side):
        torch.zeros(1, device="cuda").add_(1)
    torch.cuda.synchronize()
    dec = bench_decode(args.steps, args.warmup)
    mixed = None if args.no_prefill else bench_mixed_varlen(side=side)
    tiny = None if args.no_prefill else bench_tiny_prefill()
    pre = None if args.no_prefill else bench_prefill(args.prefill_steps, 50)
    long_kv = None if args.no_prefill else bench_prefill_long_kv(max(10, args.prefill_steps // 2), 20)
    groups = None if args.no_prefill else bench_prefill_groups()
    router = None if args.no_prefill else bench_router(200, 50)
    epilogue = None if args.no_prefill else bench_epilogue(200, 50)
    ragged = None if args.no_prefill else bench_ragged_decode()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dec["wl"], pre["wl"] if pre else __import__(
            "gqa_attention_head_amd.workloads", fromlist=["x"]).causal_prefill(), tiny)

    kernel_gbs = dec["kv_bytes"] / (dec["split_ms_mean"] * 1e-3) / 1e9
    traffic = measured_traffic()
    hbm_ctx = context_hbm()
    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "wall_ms_per_step": round(dec["wall_ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dec["workload"], "batch": dec["batch"], "kv_len": dec["kv_len"],
                   "num_q_heads": 64, "num_kv_heads": 8, "head_dim": 64,
                   "kv_chunk": dec["chunk"], "num_chunks": dec["num_chunks"],
                   "kv_copies_rotated": KV_COPIES, "parallelism": "single-gpu"},
        "hbm_frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
        "step_ms_p10_p50_p90": [round(x, 5) for x in dec["step_ms_p10_p50_p90"]],
        "context_hbm": hbm_ctx,
        "graph_replay": {"ms_per_step": round(dec["graph_ms_per_step"], 5),
                         "value": round(dec["kv_bytes"] / (dec["graph_ms_per_step"] * 1e-3) / 1e9, 2),
                         "unit": "GB/s",
                         "host_synced_ms_per_step": {k: round(v, 5) for k, v in dec["sync_ms"].items()}},
        "roofline": {"kernel": "decode_split_mfma<8, 2, 8, false>", "bound": "hbm",
                     "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic.get("decode"),
                     "algorithmic_bytes": dec["kv_bytes"],
                     "launch_ms_mean": round(dec["split_ms_mean"], 5),
                     "frac_of_read_probe": round(kernel_gbs / hbm_ctx["read_probe_gbs"], 4)},
    }
    if pre is not None:
        line["prefill"] = {
            "workload": pre["workload"], "value": round(pre["tflops"], 2), "unit": "TFLOP/s",
            "ms": round(pre["ms_mean"], 4), "flops": pre["flops"],
            "ms_p10_p50_p90": [round(x, 4) for x in pre["ms_p10_p50_p90"]],
            "roofline": {"kernel": "prefill_mfma<8, false, false>", "bound": "mfma",
                         "achieved": round(pre["tflops"], 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pre["tflops"] / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic.get("prefill"), "algorithmic_flops": pre["flops"]},
            "context_vendor_gemm_bf16_8192": {
                "tflops": round(pre["gemm_tflops"], 1),
                "frac_of_peak": round(pre["gemm_tflops"] / BF16_PEAK_TFLOPS, 4),
                "prefill_over_gemm": round(pre["tflops"] / pre["gemm_tflops"], 4)}}
    if long_kv is not None:
        line["prefill_long_kv"] = long_kv
    if groups is not None:
        line["prefill"]["other_group_sizes"] = groups
    if router is not None:
        router["roofline"]["traffic"] = traffic.get("router")
        line["router"] = router
    if epilogue is not None:
        epilogue["roofline"]["traffic"] = traffic.get("epilogue")
        line["qkv_epilogue"] = epilogue
    if ragged is not None:
        line["ragged_decode"] = ragged
    if tiny is not None:
        line["tiny_prefill_fp32"] = {k: v for k, v in tiny.items() if not k.startswith("_")}
    if mixed is not None:
        line["mixed_varlen"] = mixed
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
