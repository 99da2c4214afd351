"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every comparison is element by element on the same seeded inputs; bf16 paths
to max-abs 2e-2 / mean-abs 2e-3, fp32 paths to max-abs 1e-5.  Full-size
workloads are compared on every output where the oracle finishes in seconds,
otherwise on sampled query rows (each computed by the oracle on its own).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import gqa_attention_head_amd as sa
from gqa_attention_head_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

import gpu_helpers as H  # noqa: E402

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _sample_rows(wl, per_seq=24, seed=0):
    """Rows at tile edges, the first and last rows, and random rows of every sequence."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(wl.batch):
        lo, lq = int(wl.cu_q[b]), int(wl.seqlens_q[b])
        fixed = {0, 1, 31, 32, 33, 63, 64, 65, lq // 2, lq - 2, lq - 1}
        cand = sorted(x for x in fixed if 0 <= x < lq)
        extra = rng.choice(lq, size=min(per_seq, lq), replace=False).tolist() if lq else []
        rows += [lo + x for x in sorted(set(cand) | set(extra))]
    return np.array(rows, dtype=np.int64)


# ---------------------------------------------------------------- the five workloads

def test_tiny_prefill_fp32(orc):
    wl = W.workload(1)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=False)
    H.assert_lse_close(lse, ref_lse, bf16=False)


def test_batched_decode_split8(orc):
    wl = W.workload(2)
    dev = H.Device(wl)
    out, lse, pm, pd, pa = H.run_decode(dev, wl.kv_chunk, return_partials=True)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref[:, :, :], bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)
    # chunk states (m, d, acc): compare what is unique, acc/d and m + ln d
    nch = pm.shape[2]
    om, od, oa = orc.partials(wl.q32, wl.k32, wl.v32, wl.sinks, wl.cu_k, wl.sm_scale,
                              wl.kv_chunk, nch, nthreads=NTHREADS)
    H.assert_close(pa / pd[..., None], oa / od[..., None], bf16=True, what="chunk acc/d")
    np.testing.assert_allclose(pm + np.log(pd), om + np.log(od), atol=H.BF16_LSE)


def test_causal_prefill_4x4096_sampled(orc):
    wl = W.workload(3)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    rows = _sample_rows(wl, per_seq=24)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)
    assert np.all(np.isfinite(out))


def test_ragged_long_decode(orc):
    wl = W.workload(4)
    dev = H.Device(wl)
    out, lse = H.run_decode(dev, wl.kv_chunk)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("permute", [False, True])
def test_mixed_varlen_prefill_call(orc, permute):
    wl = W.mixed_varlen(permute=permute)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    rows = _sample_rows(wl, per_seq=16)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)


def test_mixed_varlen_decode_rows_via_split(orc):
    """The 12 single-token sequences of the mixed batch through split + merge agree with
    the oracle and with the prefill call's rows."""
    wl = W.mixed_varlen()
    dev = H.Device(wl)
    first = 4
    q_rows = wl.cu_q[first:-1]
    q = dev.q[torch.from_numpy(q_rows.astype(np.int64)).cuda()].contiguous()
    cu_k = dev.cu_k[first:].contiguous()
    max_lk = int(wl.seqlens_k[first:].max())
    out, lse = H.run_decode(dev, 2048, q=q, cu_k=cu_k, max_lk=max_lk)
    ref, ref_lse = orc.workload(wl, rows=q_rows.astype(np.int64), nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)
    pout, _ = H.run_prefill(dev)
    assert np.abs(pout[q_rows] - out).max() <= 2 * H.BF16_MAX_ABS


def test_mixed_varlen_two_streams(orc):
    """The mixed batch as a prefill call over its 4 chunks on the current stream and a
    decode call over its 12 single-token sequences on a second stream, writing disjoint
    rows of one output (the overlapped form bench.py times), agrees with the oracle."""
    wl = W.mixed_varlen()
    dev = H.Device(wl)
    npre = 4
    r0 = int(wl.cu_q[npre])
    lq, lk = wl.seqlens_q, wl.seqlens_k
    out = torch.full_like(dev.q, float("nan"))
    ws = sa.DecodeWorkspace(len(lq) - npre, wl.num_q_heads, -(-int(lk[npre:].max()) // 2048),
                            wl.head_dim, dev.q.device)
    side = torch.cuda.Stream()
    for _ in range(3):  # repeated, as timed
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            sa.decode(dev.q[r0:], dev.k, dev.v, dev.sinks, dev.cu_k[npre:], int(lk[npre:].max()),
                      2048, wl.sm_scale, workspace=ws, out=out[r0:])
        sa.prefill(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q[:npre + 1], dev.cu_k[:npre + 1],
                   int(lq[:npre].max()), int(lk[:npre].max()), wl.sm_scale, causal=True, out=out)
        main.wait_stream(side)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rows = _sample_rows(wl, per_seq=16)
    ref, _ = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(got[rows], ref, bf16=True)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("chunk", [4096, 2048, 512, 64, 37, 1])
def test_split_invariance(orc, chunk):
    wl = W.random_case(21, batch=3, hq=16, hkv=2, max_k=3000, decode=True,
                       sink_values=[-np.inf, -20, 0, 20] * 4)
    dev = H.Device(wl)
    out, lse = H.run_decode(dev, chunk)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_group_sizes_prefill(orc, group, dtype):
    wl = W.random_case(30 + group, dtype=dtype, batch=3, hq=2 * group, hkv=2, max_q=150,
                       max_k=400)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=dtype == "bf16")
    H.assert_lse_close(lse, ref_lse, bf16=dtype == "bf16")


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_group_sizes_decode(orc, group, dtype):
    wl = W.random_case(50 + group, dtype=dtype, batch=4, hq=2 * group, hkv=2, max_k=700,
                       decode=True)
    dev = H.Device(wl)
    out, lse = H.run_decode(dev, 128)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=dtype == "bf16")
    H.assert_lse_close(lse, ref_lse, bf16=dtype == "bf16")


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_prefill_over_cache(orc, causal):
    """L_q < L_k with ragged tails, both maskings."""
    wl = W.make_workload("ragged", dtype="bf16", kind="prefill", seqlens_q=[1, 31, 33, 100, 65],
                         seqlens_k=[1, 200, 33, 357, 64 + 65], num_q_heads=16, num_kv_heads=2,
                         head_dim=64, seed=61, causal=causal)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("group", [1, 3, 8, 16, 24])
@pytest.mark.parametrize("extra", [(0, 150, 33, 300, 700), (0, 150, 33, 300, 5000)])
def test_prefill_over_caches_group_sizes(orc, group, extra):
    """Causal chunks over caches of different lengths (not multiples of the 32-row
    block) for several group sizes, with workgroups of one or several query blocks
    and head slices; short and long caches."""
    lq = [37, 100, 256, 1, 64]
    wl = W.make_workload("over_caches", dtype="bf16", kind="prefill", seqlens_q=lq,
                         seqlens_k=[a + b for a, b in zip(lq, extra)], num_q_heads=2 * group,
                         num_kv_heads=2, head_dim=64, seed=70 + group, causal=True)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_empty_and_single_key_sequences(orc, dtype):
    """Decode with L = 0 (chunk 0 holds only the sink), L = 1, and a sink of -inf with no keys."""
    wl = W.make_workload("empties", dtype=dtype, kind="decode", seqlens_q=[1, 1, 1, 1],
                         seqlens_k=[0, 1, 0, 5], num_q_heads=8, num_kv_heads=2, head_dim=64,
                         seed=62, causal=False,
                         sink_values=[-np.inf, 0.5, -np.inf, 3.0, -1.0, -np.inf, 20.0, -20.0])
    dev = H.Device(wl)
    out, lse = H.run_decode(dev, 4)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=dtype == "bf16")
    H.assert_lse_close(lse, ref_lse, bf16=dtype == "bf16")
    # the same through the prefill entry point (non-causal, one query per sequence)
    out2, lse2 = H.run_prefill(dev)
    H.assert_close(out2, ref, bf16=dtype == "bf16")
    H.assert_lse_close(lse2, ref_lse, bf16=dtype == "bf16")


def test_log2_domain_sinks(orc):
    """Large sinks next to large scores: a kernel that seeded the base-2 running max with the
    natural-log sink (or scaled the sink by sm_scale) would be far off here."""
    rng = np.random.default_rng(63)
    wl = W.make_workload("log2trap", dtype="bf16", kind="prefill", seqlens_q=[40, 1],
                         seqlens_k=[40, 300], num_q_heads=8, num_kv_heads=1, head_dim=64, seed=63,
                         causal=True, sink_values=[20.0, -20.0, 12.0, 5.0, 0.0, -5.0, 8.0, 15.0],
                         rng=rng)
    # scale q up so the scores reach the sinks' range
    wl.q16 = W.bf16_round(wl.q32 * 4.0)
    wl.q32 = W.bf16_widen(wl.q16)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)
    dout, dlse = H.run_decode(dev, 64, q=dev.q[torch.tensor([39, 40]).cuda()].contiguous())
    dref, dref_lse = orc.workload(wl, rows=np.array([39, 40]), nthreads=NTHREADS)
    H.assert_close(dout, dref, bf16=True)
    H.assert_lse_close(dlse, dref_lse, bf16=True)


@pytest.mark.parametrize("ramp", ["rising", "falling"])
def test_running_max_growth(orc, ramp):
    """Scores whose scale grows (or shrinks) along the keys: with a rising ramp each row's
    maximum keeps climbing far past the running one (many rescales, also mid-sequence and
    after a sink that was the maximum); with a falling ramp the first tile sets the
    maximum for good.  Sinks cover -inf, large negative, zero and large positive."""
    rng = np.random.default_rng(65)
    lq, lk = 96, 700
    wl = W.make_workload(f"ramp_{ramp}", dtype="bf16", kind="prefill", seqlens_q=[lq, 1],
                         seqlens_k=[lk, lk], num_q_heads=8, num_kv_heads=2, head_dim=64, seed=65,
                         causal=True,
                         sink_values=[float("-inf"), -20.0, 0.0, 20.0, 3.0, float("-inf"), 40.0, -3.0],
                         rng=rng)
    j = np.arange(wl.k32.shape[0]) % lk
    f = 1.0 + 24.0 * j / lk if ramp == "rising" else 25.0 - 24.0 * j / lk
    wl.k16 = W.bf16_round((wl.k32 * f[:, None, None]).astype(np.float32))
    wl.k32 = W.bf16_widen(wl.k16)
    wl.q16 = W.bf16_round(wl.q32 * 2.0)
    wl.q32 = W.bf16_widen(wl.q16)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)
    _, _, _, mout, mlse = run_prefill_split(dev, 128)
    H.assert_close(mout, ref, bf16=True)
    H.assert_lse_close(mlse, ref_lse, bf16=True)


def test_prefill_rows_equal_decode(orc):
    """Row i of a causal prefill equals a decode of that query over its visible keys."""
    wl = W.make_workload("pd", dtype="bf16", kind="prefill", seqlens_q=[70], seqlens_k=[250],
                         num_q_heads=8, num_kv_heads=1, head_dim=64, seed=64, causal=True)
    dev = H.Device(wl)
    out, _ = H.run_prefill(dev)
    for i in (0, 33, 69):
        n = 250 - 70 + i + 1
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        dout, _ = H.run_decode(dev, 64, q=dev.q[i:i + 1].contiguous(), cu_k=cu, max_lk=n)
        assert np.abs(dout[0] - out[i]).max() <= 2 * H.BF16_MAX_ABS


# ---------------------------------------------------------------- one-call decode

def test_decode_call_batched(orc):
    """The 32 x 4096 decode (8 chunks) through sink_attn_decode, twice in a row with
    one workspace: both calls agree with the oracle."""
    wl = W.workload(2)
    dev = H.Device(wl)
    ws = sa.DecodeWorkspace(wl.batch, wl.num_q_heads, 8)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    for _ in range(2):
        out, lse = H.run_decode_call(dev, wl.kv_chunk, workspace=ws)
        H.assert_close(out, ref, bf16=True)
        H.assert_lse_close(lse, ref_lse, bf16=True)


def test_decode_call_ragged_long(orc):
    """64 chunk slots per sequence, ragged lengths up to 131072 keys."""
    wl = W.workload(4)
    dev = H.Device(wl)
    out, lse = H.run_decode_call(dev, wl.kv_chunk)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 64])
@pytest.mark.parametrize("chunk", [37, 256, 4096])
def test_decode_call_cases(orc, group, chunk):
    wl = W.random_case(70 + group, batch=5, hq=2 * group, hkv=2, max_k=1500, decode=True,
                       sink_values=([-np.inf, 20.0, -20.0, 0.5] * group)[:2 * group])
    dev = H.Device(wl)
    ws = sa.DecodeWorkspace(wl.batch, wl.num_q_heads, max(1, -(-dev.max_lk // chunk)))
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    for _ in range(2):
        out, lse = H.run_decode_call(dev, chunk, workspace=ws)
        H.assert_close(out, ref, bf16=True)
        H.assert_lse_close(lse, ref_lse, bf16=True)


def test_decode_call_empty_sequences(orc):
    wl = W.make_workload("empties_call", dtype="bf16", kind="decode", seqlens_q=[1] * 4,
                         seqlens_k=[0, 1, 0, 70], num_q_heads=8, num_kv_heads=1, head_dim=64,
                         seed=77, causal=False,
                         sink_values=[-np.inf, 0.5, -np.inf, 3.0, -1.0, -np.inf, 20.0, -20.0])
    dev = H.Device(wl)
    out, lse = H.run_decode_call(dev, 32)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


# ---------------------------------------------------------------- graph-captured decode

def test_decode_graph_replays(orc):
    """A captured decode call replayed several times, with eager work and host
    synchronisation between replays: every replay equals the eager call bit for bit,
    also after new inputs are copied into the captured buffers."""
    wl = W.random_case(91, batch=6, hq=16, hkv=2, max_k=2500, decode=True,
                       sink_values=[-np.inf, 20.0, -20.0, 0.5] * 4)
    dev = H.Device(wl)
    chunk = 512
    g = sa.DecodeGraph(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk, wl.sm_scale)
    eager = sa.decode(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk, wl.sm_scale,
                      return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(eager[0].float().cpu().numpy().astype(np.float64), ref, bf16=True)
    for i in range(3):
        out, lse = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1]), f"replay {i} differs"
        _ = (torch.randn(1024, device="cuda") * 2).sum().item()  # eager work in between
    # new queries written into the captured buffer
    q2 = torch.flip(dev.q, dims=[0]).contiguous()
    dev.q.copy_(q2)
    eager2 = sa.decode(dev.q, dev.k, dev.v, dev.sinks, dev.cu_k, dev.max_lk, chunk, wl.sm_scale,
                       return_lse=True)
    for i in range(2):
        out, lse = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager2[0]) and torch.equal(lse, eager2[1]), f"replay {i} (new q)"


# ---------------------------------------------------------------- split-KV prefill

def run_prefill_split(dev: "H.Device", chunk: int, causal=None):
    wl = dev.wl
    causal = wl.causal if causal is None else causal
    nch = max(1, -(-dev.max_lk // chunk))
    pm, pd, pa = sa.prefill_split(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q, dev.cu_k,
                                  dev.max_lq, dev.max_lk, chunk, wl.sm_scale, causal=causal,
                                  max_num_chunks=nch)
    out, lse = sa.merge_rows(pm, pd, pa, out_dtype=dev.dtype, return_lse=True)
    torch.cuda.synchronize()
    return pm, pd, pa, out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_split_spare_chunk_slots(orc, dtype):
    """max_num_chunks three above what the keys need: the slots past each sequence's
    last chunk hold the empty state (m = -inf, d = 0, acc = 0), every slot merges to the
    plain definition, and decode split + merge with spare slots does too."""
    bf16 = dtype == "bf16"
    wl = W.random_case(140, dtype=dtype, batch=3, hq=16, hkv=2, max_q=90, max_k=700,
                       sink_values=[-np.inf, 20.0, -20.0, 0.5] * 4)
    dev = H.Device(wl)
    chunk = 128
    need = -(-dev.max_lk // chunk)
    pm, pd, pa = sa.prefill_split(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q, dev.cu_k,
                                  dev.max_lq, dev.max_lk, chunk, wl.sm_scale, causal=True,
                                  max_num_chunks=need + 3)
    out, lse = sa.merge_rows(pm, pd, pa, out_dtype=dev.dtype, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out.float().cpu().numpy().astype(np.float64), ref, bf16=bf16)
    H.assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_lse, bf16=bf16)
    pm, pd, pa = pm.cpu().numpy(), pd.cpu().numpy(), pa.cpu().numpy()
    for b in range(wl.batch):
        rows = slice(int(wl.cu_q[b]), int(wl.cu_q[b + 1]))
        first_spare = max(1, -(-int(wl.seqlens_k[b]) // chunk))
        assert np.all(pm[rows, :, first_spare:] == -np.inf)
        assert np.all(pd[rows, :, first_spare:] == 0.0)
        assert np.all(pa[rows, :, first_spare:, :] == 0.0)
    # the one-call decode with spare chunk slots (each sequence's last query row)
    last = (wl.cu_q[1:] - 1).astype(np.int64)
    qd = dev.q[torch.from_numpy(last).cuda()].contiguous()
    dout, dlse = H.run_decode_call(dev, chunk, q=qd, max_num_chunks=need + 3)
    H.assert_close(dout, ref[last], bf16=bf16)
    H.assert_lse_close(dlse, ref_lse[last], bf16=bf16)


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 64])
@pytest.mark.parametrize("chunk", [64, 100, 1024])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_split_cases(orc, group, chunk, causal):
    """Split-KV prefill + row merge against the plain definition: several tiles per
    chunk, ragged chunk ends, chunks not aligned to the 64-key tiles, L_q < L_k."""
    wl = W.random_case(110 + group, batch=3, hq=2 * group, hkv=2, max_q=150, max_k=900,
                       causal=causal, sink_values=([-np.inf, 20.0, -20.0, 0.5] * group)[:2 * group])
    dev = H.Device(wl)
    _, _, _, out, lse = run_prefill_split(dev, chunk)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


@pytest.mark.parametrize("chunk", [64, 96])
def test_prefill_split_fp32(orc, chunk):
    wl = W.random_case(131, dtype="fp32", batch=2, hq=8, hkv=2, max_q=100, max_k=400)
    dev = H.Device(wl)
    _, _, _, out, lse = run_prefill_split(dev, chunk)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=False)
    H.assert_lse_close(lse, ref_lse, bf16=False)


@pytest.mark.parametrize("group", [8, 3])
def test_prefill_split_chunk_states(orc, group):
    """Each chunk state against the definition restricted to the chunk: the keys of
    chunk c the row may see, with the sink in chunk 0 only; chunks a row cannot see
    hold (m = -inf, d = 0, acc = 0)."""
    chunk = 128
    wl = W.random_case(140 + group, batch=2, hq=2 * group, hkv=2, max_q=200, max_k=700,
                       sink_values=([-np.inf, 1.5, -20.0, 0.5] * group)[:2 * group])
    dev = H.Device(wl)
    pm, pd, pa, _, _ = run_prefill_split(dev, chunk)
    pm, pd, pa = (t.cpu().numpy().astype(np.float64) for t in (pm, pd, pa))
    nch = pm.shape[2]
    rng = np.random.default_rng(5)
    rows = rng.choice(int(wl.cu_q[-1]), 12, replace=False)
    for r in rows:
        b = int(np.searchsorted(wl.cu_q, r, side="right") - 1)
        i = int(r - wl.cu_q[b])
        lq, lk = int(wl.seqlens_q[b]), int(wl.seqlens_k[b])
        vis = lk - lq + i + 1 if wl.causal else lk
        for c in range(nch):
            lo, hi = c * chunk, min((c + 1) * chunk, max(vis, 0))
            n = max(0, hi - lo)
            kk = wl.k32[wl.cu_k[b] + lo:wl.cu_k[b] + lo + n]
            vv = wl.v32[wl.cu_k[b] + lo:wl.cu_k[b] + lo + n]
            sinks = wl.sinks if c == 0 else np.full_like(wl.sinks, -np.inf)
            ref, ref_lse = orc.attention(wl.q32[r:r + 1], kk, vv, sinks, np.array([0, 1]),
                                         np.array([0, n]), wl.sm_scale, causal=False,
                                         nthreads=1)
            for h in range(wl.num_q_heads):
                m, d = pm[r, h, c], pd[r, h, c]
                if not np.isfinite(ref_lse[0, h]):
                    assert m == -np.inf and np.all(pa[r, h, c] == 0.0), (r, h, c)
                    if c > 0:
                        assert d == 0.0, (r, h, c)
                    continue
                got_lse = m + np.log(d)
                assert abs(got_lse - ref_lse[0, h]) <= H.BF16_LSE, (r, h, c, got_lse, ref_lse[0, h])
                assert np.abs(pa[r, h, c] / d - ref[0, h]).max() <= H.BF16_MAX_ABS, (r, h, c)


def test_prefill_split_mixed_varlen(orc):
    """Workload 5 (prefill chunks over cached keys and single-token decodes, sinks from
    {-inf, -20, 0, +20, N(0,1)}) through the split prefill with 1024-key chunks."""
    wl = W.workload(5)
    dev = H.Device(wl)
    _, _, _, out, lse = run_prefill_split(dev, 1024)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(int(wl.cu_q[-1]), 256, replace=False))
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)


def test_prefill_split_matches_unsplit():
    """The split and unsplit prefill agree on the 4 x 4096 causal workload (sampled
    rows), within the bf16 tolerance (split-invariance of the method)."""
    wl = W.workload(3)
    dev = H.Device(wl)
    _, _, _, out, lse = run_prefill_split(dev, 1024)
    full, full_lse = sa.prefill(dev.q, dev.k, dev.v, dev.sinks, dev.cu_q, dev.cu_k, dev.max_lq,
                                dev.max_lk, wl.sm_scale, causal=True, return_lse=True)
    torch.cuda.synchronize()
    full = full.float().cpu().numpy().astype(np.float64)
    full_lse = full_lse.cpu().numpy().astype(np.float64)
    assert np.abs(out - full).max() <= H.BF16_MAX_ABS
    assert np.abs(lse - full_lse).max() <= 1e-4


# ---------------------------------------------------------------- long inputs

def test_long_single_sequence_prefill_sampled(orc):
    """One 32768-token causal sequence (64/8 heads): the longest rows of the path's
    prefill kernel, checked on sampled rows including the last ones."""
    wl = W.make_workload("long_prefill", dtype="bf16", kind="prefill", seqlens_q=[32768],
                         seqlens_k=[32768], num_q_heads=64, num_kv_heads=8, head_dim=64, seed=71,
                         causal=True)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    rows = np.array([0, 63, 64, 4095, 16384, 32766, 32767], dtype=np.int64)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)
    assert np.all(np.isfinite(out))


def test_max_batch_decode_and_prefill(orc):
    """The largest batch the entry points accept (65535 sequences), ragged 1-3 keys each,
    G = 8 on one KV head: the decode split + merge (chunk 2, so up to 2 chunks) and the
    prefill of the same single-token rows, checked on sampled sequences."""
    batch = 65535
    rng = np.random.default_rng(81)
    lk = rng.integers(1, 3, size=batch, endpoint=True).tolist()
    wl = W.make_workload("max_batch", dtype="bf16", kind="decode", seqlens_q=[1] * batch,
                         seqlens_k=lk, num_q_heads=8, num_kv_heads=1, head_dim=64, seed=82,
                         causal=False, sink_values=[-np.inf, -2.0, 0.0, 1.0, 2.0, 4.0, 0.5, -1.0])
    dev = H.Device(wl)
    rows = np.array([0, 1, 2, 1000, 32767, 65533, 65534], dtype=np.int64)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    out, lse = H.run_decode(dev, 2)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)
    assert np.all(np.isfinite(out))
    pout, plse = H.run_prefill(dev, causal=False)
    H.assert_close(pout[rows], ref, bf16=True)
    H.assert_lse_close(plse[rows], ref_lse, bf16=True)


def test_long_kv_split_prefill_bench_shape(orc):
    """The benchmark's chunked prefill: 256 new tokens over 131072 keys (64/8 heads),
    16384-key chunks, split pass then row merge; sampled rows against the oracle."""
    wl = W.make_workload("long_kv", dtype="bf16", kind="prefill", seqlens_q=[256],
                         seqlens_k=[131072], num_q_heads=64, num_kv_heads=8, head_dim=64,
                         seed=72, causal=True)
    dev = H.Device(wl)
    _, _, _, out, lse = run_prefill_split(dev, 16384)
    rows = np.array([0, 1, 31, 32, 128, 254, 255], dtype=np.int64)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)


# ---------------------------------------------------------------- many short sequences

def test_many_short_sequences_prefill(orc):
    """2000 causal sequences of 1..40 tokens over 0..60 cached keys each (16/2 heads):
    the packed varlen indexing at a large batch, every row checked."""
    wl = W.random_case(101, batch=2000, hq=16, hkv=2, max_q=40, max_k=100)
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


def test_many_short_sequences_decode(orc):
    """4096 single-token sequences of 1..300 keys (16/2 heads), 64-key chunks, through
    the one-call decode; every sequence checked."""
    wl = W.random_case(102, batch=4096, hq=16, hkv=2, max_k=300, decode=True)
    dev = H.Device(wl)
    out, lse = H.run_decode_call(dev, 64)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)


# ---------------------------------------------------------------- seeded random configurations

@pytest.mark.parametrize("seed", range(24))
def test_random_configurations(orc, seed):
    """Seeded random shapes: group size, KV heads, batch, lengths, causal or not, dtype and
    chunk lengths drawn per seed; prefill, split prefill + row merge and one-call decode
    each against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    group = int(rng.choice([1, 2, 3, 4, 8, 16]))
    hkv = int(rng.integers(1, 4))
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    causal = bool(rng.random() < 0.7)
    batch = int(rng.integers(1, 6))
    max_q = int(rng.integers(1, 150))
    max_k = max_q + int(rng.integers(0, 300))
    wl = W.random_case(2000 + seed, dtype=dtype, batch=batch, hq=hkv * group, hkv=hkv,
                       max_q=max_q, max_k=max_k, causal=causal,
                       sink_sigma=float(rng.choice([1.0, 4.0])))
    bf16 = dtype == "bf16"
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    out, lse = H.run_prefill(dev)
    H.assert_close(out, ref, bf16=bf16)
    H.assert_lse_close(lse, ref_lse, bf16=bf16)
    chunk = int(rng.integers(1, max(2, dev.max_lk + 1)))
    _, _, _, sout, slse = run_prefill_split(dev, chunk)
    H.assert_close(sout, ref, bf16=bf16)
    H.assert_lse_close(slse, ref_lse, bf16=bf16)
    # decode: each sequence's last query row, which sees all of its keys either way
    last = (wl.cu_q[1:] - 1).astype(np.int64)
    qd = dev.q[torch.from_numpy(last).cuda()].contiguous()
    dout, dlse = H.run_decode_call(dev, int(rng.integers(1, 200)), q=qd)
    H.assert_close(dout, ref[last], bf16=bf16)
    H.assert_lse_close(dlse, ref_lse[last], bf16=bf16)


# ---------------------------------------------------------------- short query rows in prefill

@pytest.mark.parametrize("group", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_short_query_rows(orc, group, causal):
    """Sequences of at most 16 / G query rows (the prefill call's decode-style path: the
    workgroup's waves split the keys and combine their states in LDS), mixed with longer
    chunks in one call, over caches from 0 to 9000 keys; every output element."""
    rows = max(1, 16 // group)
    lq = [1, rows, rows, 1, 40, rows, 1]
    lk = [5000, rows + 9000, rows, 1, 700, rows + 37, 0 if not causal else 1]
    hkv = 2
    wl = W.make_workload(f"short_rows_g{group}", dtype="bf16", kind="prefill", seqlens_q=lq,
                         seqlens_k=lk, num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=64,
                         seed=900 + group, causal=causal,
                         sink_values=([-np.inf, 20.0, -20.0, 0.5, 3.0] * group)[:hkv * group])
    dev = H.Device(wl)
    out, lse = H.run_prefill(dev)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    H.assert_close(out, ref, bf16=True)
    H.assert_lse_close(lse, ref_lse, bf16=True)
