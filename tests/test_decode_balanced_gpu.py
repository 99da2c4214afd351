"""GPU parity of the one-call decode with proportional blocks (``sink_attn_decode`` with
kv_chunk_size = 0): each sequence is cut into a number of blocks proportional to its
length, about one workgroup per compute unit in all, whatever the sequence lengths.  Each case is compared element by element
with the fp64 oracle; the partial-state buffers sit between NaN guard bands that
must stay untouched."""
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


class GuardedWorkspace:
    """A decode workspace whose three state buffers are views into NaN-poisoned
    buffers with guard bands on both sides."""

    def __init__(self, batch, hq, slots, d=64):
        self.batch, self.num_q_heads, self.head_dim, self.max_num_chunks = batch, hq, d, slots
        self._m = H.guarded((batch, hq, slots), torch.float32)
        self._d = H.guarded((batch, hq, slots), torch.float32)
        self._a = H.guarded((batch, hq, slots, d), torch.float32)
        self.partials = (self._m[0], self._d[0], self._a[0])

    def check(self):
        for view, buf in (self._m, self._d, self._a):
            H.check_guard(buf, view.numel())


def balanced(dev, q=None, cu_k=None, max_lk=None, slots=None, chunk=0, calls=1):
    """sink_attn_decode with proportional blocks (chunk 0) into a guarded workspace."""
    wl = dev.wl
    q = dev.q if q is None else q
    cu_k = dev.cu_k if cu_k is None else cu_k
    max_lk = dev.max_lk if max_lk is None else max_lk
    batch = cu_k.numel() - 1
    if slots is None:
        slots = sa.balanced_slots(batch, wl.num_q_heads, wl.head_dim)
    ws = GuardedWorkspace(batch, wl.num_q_heads, slots, wl.head_dim)
    res = []
    for _ in range(calls):
        res.append(H.run_decode_call(dev, chunk, q=q, cu_k=cu_k, max_lk=max_lk, workspace=ws))
    ws.check()
    return res


def check(res, ref, ref_lse, bf16=True):
    for out, lse in res:
        H.assert_close(out, ref, bf16=bf16)
        H.assert_lse_close(lse, ref_lse, bf16=bf16)


def test_balanced_batched_decode(orc):
    """The 32 x 4096 decode: proportional blocks give the same result as the 8 chunks."""
    wl = W.workload(2)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, calls=2), ref, ref_lse)
    check(balanced(dev, slots=8), ref, ref_lse)


def test_balanced_ragged_long_decode(orc):
    """The long-context ragged decode (8 sequences of 1024-131072 keys), every output."""
    wl = W.workload(4)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, calls=2), ref, ref_lse)
    check(balanced(dev, slots=64), ref, ref_lse)


def test_balanced_mixed_varlen_decodes(orc):
    """The mixed batch's 12 single-token sequences (1024-32768 keys)."""
    wl = W.mixed_varlen()
    dev = H.Device(wl)
    first = 4
    q_rows = wl.cu_q[first:-1].astype(np.int64)
    q = dev.q[torch.from_numpy(q_rows).cuda()].contiguous()
    cu_k = dev.cu_k[first:].contiguous()  # offsets start at the first decode's keys
    max_lk = int(wl.seqlens_k[first:].max())
    ref, ref_lse = orc.workload(wl, rows=q_rows, nthreads=NTHREADS)
    check(balanced(dev, q=q, cu_k=cu_k, max_lk=max_lk), ref, ref_lse)


@pytest.mark.parametrize("lengths", [
    [0, 1, 0, 70],                      # empty sequences between others
    [0, 0, 1],                          # almost no keys
    [5000, 0],                          # empty last sequence
    [0, 3000, 1, 1, 2, 4000],           # long and one-key sequences side by side
    [1] * 300,                          # more sequences than block columns
    [129, 127, 128, 256, 255, 257],     # around the 32- and 64-key tile sizes
])
def test_balanced_empty_and_short_sequences(orc, lengths):
    wl = W.make_workload("balanced_edges", dtype="bf16", kind="decode",
                         seqlens_q=[1] * len(lengths), seqlens_k=lengths, num_q_heads=8,
                         num_kv_heads=1, head_dim=64, seed=len(lengths) + sum(lengths),
                         causal=False,
                         sink_values=[-np.inf, 0.5, -np.inf, 3.0, -1.0, -np.inf, 20.0, -20.0])
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, calls=2), ref, ref_lse)


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 17, 24, 32, 64])
def test_balanced_group_sizes(orc, group):
    """Every group size: one wave per KV head, or per slice of its query heads."""
    hkv = 2 if group <= 16 else 1
    wl = W.random_case(300 + group, batch=7, hq=hkv * group, hkv=hkv, max_k=6000, decode=True,
                       sink_values=([-np.inf, 20.0, -20.0, 0.5] * group)[:hkv * group])
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev), ref, ref_lse)


@pytest.mark.parametrize("slots", [2, 3, 5, 1])
def test_balanced_few_slots(orc, slots):
    """Few state slots per sequence: the blocks grow so that no sequence gets more
    blocks than there are slots (one slot: one block per sequence)."""
    wl = W.random_case(350 + slots, batch=6, hq=16, hkv=2, max_k=9000, decode=True)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, slots=slots), ref, ref_lse)


def test_balanced_fp32_takes_fixed_chunks(orc):
    """fp32 inputs (vector-ALU path): chunk 0 becomes the finest fixed chunks the slots
    allow, with the fp32 tolerance."""
    wl = W.random_case(361, dtype="fp32", batch=5, hq=8, hkv=2, max_k=700, decode=True)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, slots=7), ref, ref_lse, bf16=False)


def test_balanced_offsets_not_from_zero(orc):
    """Sequence offsets that start inside the key buffer (cu_seqlens_k[0] > 0)."""
    wl = W.random_case(362, batch=9, hq=16, hkv=2, max_k=5000, decode=True)
    dev = H.Device(wl)
    sub = slice(3, None)
    q = dev.q[3:].contiguous()
    cu_k = dev.cu_k[3:].contiguous()
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev, q=q, cu_k=cu_k, max_lk=int(wl.seqlens_k[sub].max())),
          ref[3:], ref_lse[3:])


def test_balanced_many_short_sequences(orc):
    """4096 single-token sequences of 1..300 keys (16/2 heads)."""
    wl = W.random_case(102, batch=4096, hq=16, hkv=2, max_k=300, decode=True)
    dev = H.Device(wl)
    ref, ref_lse = orc.workload(wl, nthreads=NTHREADS)
    check(balanced(dev), ref, ref_lse)


def test_balanced_max_batch(orc):
    """65535 sequences of 1-3 keys: the block-to-sequence search over the largest batch
    (three narrowing rounds), sampled sequences against the oracle."""
    batch = 65535
    rng = np.random.default_rng(83)
    lk = rng.integers(1, 3, size=batch, endpoint=True).tolist()
    wl = W.make_workload("max_batch_balanced", dtype="bf16", kind="decode",
                         seqlens_q=[1] * batch, seqlens_k=lk, num_q_heads=8, num_kv_heads=1,
                         head_dim=64, seed=84, causal=False,
                         sink_values=[-np.inf, -2.0, 0.0, 1.0, 2.0, 4.0, 0.5, -1.0])
    dev = H.Device(wl)
    rows = np.array([0, 1, 2, 1000, 32767, 65533, 65534], dtype=np.int64)
    ref, ref_lse = orc.workload(wl, rows=rows, nthreads=NTHREADS)
    (out, lse), = balanced(dev, slots=4)
    H.assert_close(out[rows], ref, bf16=True)
    H.assert_lse_close(lse[rows], ref_lse, bf16=True)
    assert np.all(np.isfinite(out))


def test_balanced_matches_fixed_chunks():
    """Proportional blocks and fixed chunks agree with each other to the bf16 output's
    rounding on the ragged long decode."""
    wl = W.workload(4)
    dev = H.Device(wl)
    (bout, blse), = balanced(dev)
    fout, flse = H.run_decode_call(dev, wl.kv_chunk)
    assert np.abs(bout - fout).max() <= 2 ** -7
    assert np.abs(blse - flse).max() <= 1e-4
