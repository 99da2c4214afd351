"""Seeded synthetic inputs for grouped-query attention with a per-head sink.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic, so both the CPU oracle and the HIP path can take
their inputs from it without sharing any of the method.

The shapes follow the gpt-oss attention described in "GPT-OSS on day 0"
(Perplexity, section "Attention and MLP architecture": GQA with a learned sink
per head): 64 query heads sharing 8 key/value heads, head_dim 64.  The pages
print no attention-level workload, so every tensor here is synthetic.

Recipe (shared by every workload):
  * ``rng = numpy.random.default_rng(seed)``;
  * draw order: sequence lengths, then q, k, v, then sinks;
  * q, k, v, sinks are ``rng.standard_normal(..., dtype=float32)``;
  * bf16 workloads round q, k, v to bf16 with round-to-nearest-even; the
    rounded values widen exactly back to float32, and those float32 values
    are what the oracle reads;
  * sinks are always float32 (natural-log units), sm_scale = 1/8.

Layout: token-major packed varlen ("NHD"): q is [total_q, Hq, D], k and v are
[total_k, Hkv, D]; sequence b owns q rows [cu_q[b], cu_q[b+1]) and key rows
[cu_k[b], cu_k[b+1]).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SM_SCALE = 0.125


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # modulo-2^32 sums: the top 16 bits are those of the exact sum (which is < 2^33);
    # in place, one temporary
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One synthetic attention problem, host side.

    ``q32``/``k32``/``v32`` hold the exact values both sides compute on, as
    float32.  For bf16 workloads ``q16``/``k16``/``v16`` hold the bf16 bit
    patterns the device receives.
    """

    name: str
    dtype: str                    # "fp32" or "bf16"
    kind: str                     # "prefill", "decode" or "mixed"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    cu_q: np.ndarray              # int32 [B+1]
    cu_k: np.ndarray              # int32 [B+1]
    q32: np.ndarray               # float32 [total_q, Hq, D]
    k32: np.ndarray               # float32 [total_k, Hkv, D]
    v32: np.ndarray               # float32 [total_k, Hkv, D]
    sinks: np.ndarray             # float32 [Hq]
    sm_scale: float = SM_SCALE
    causal: bool = True
    kv_chunk: int = 0             # split-KV chunk length (decode); 0 = no split
    q16: np.ndarray | None = None
    k16: np.ndarray | None = None
    v16: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.cu_q.shape[0] - 1)

    @property
    def seqlens_q(self) -> np.ndarray:
        return np.diff(self.cu_q).astype(np.int64)

    @property
    def seqlens_k(self) -> np.ndarray:
        return np.diff(self.cu_k).astype(np.int64)

    def device_arrays(self):
        """(q, k, v) as the device receives them: bf16 bits or float32."""
        if self.dtype == "bf16":
            return self.q16, self.k16, self.v16
        return self.q32, self.k32, self.v32

    def kv_bytes(self) -> int:
        """Bytes of K and V one pass over every key reads (the decode numerator)."""
        elt = 2 if self.dtype == "bf16" else 4
        return int(self.seqlens_k.sum()) * self.num_kv_heads * self.head_dim * elt * 2

    def prefill_flops(self) -> int:
        """Multiply-add flops of QK^T and PV over the causal-visible pairs only."""
        pairs = 0
        for lq, lk in zip(self.seqlens_q, self.seqlens_k):
            lq, lk = int(lq), int(lk)
            if self.causal:
                # query i sees keys 0..lk-lq+i (bottom-right alignment)
                pairs += lq * (lk - lq) + lq * (lq + 1) // 2
            else:
                pairs += lq * lk
        return 4 * self.head_dim * self.num_q_heads * pairs


def _cu(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


def _draw_qkv(rng, total_q, total_k, hq, hkv, d, dtype):
    q = rng.standard_normal((total_q, hq, d), dtype=np.float32)
    k = rng.standard_normal((total_k, hkv, d), dtype=np.float32)
    v = rng.standard_normal((total_k, hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q16, k16, v16 = bf16_round(q), bf16_round(k), bf16_round(v)
        return bf16_widen(q16), bf16_widen(k16), bf16_widen(v16), q16, k16, v16
    return q, k, v, None, None, None


def make_workload(name, *, dtype, kind, seqlens_q, seqlens_k, num_q_heads,
                  num_kv_heads, head_dim, seed, causal=True, kv_chunk=0,
                  sink_sigma=1.0, sink_values=None, rng=None, meta=None):
    """Generic builder: lengths are given, q/k/v/sinks are drawn from ``seed``."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    cu_q, cu_k = _cu(seqlens_q), _cu(seqlens_k)
    q, k, v, q16, k16, v16 = _draw_qkv(rng, int(cu_q[-1]), int(cu_k[-1]),
                                       num_q_heads, num_kv_heads, head_dim, dtype)
    if sink_values is not None:
        sinks = np.asarray(sink_values, dtype=np.float32)
    else:
        sinks = (sink_sigma * rng.standard_normal(num_q_heads, dtype=np.float32)).astype(np.float32)
    return Workload(name=name, dtype=dtype, kind=kind, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, cu_q=cu_q, cu_k=cu_k,
                    q32=q, k32=k, v32=v, sinks=sinks, causal=causal, kv_chunk=kv_chunk,
                    q16=q16, k16=k16, v16=v16, meta=dict(meta or {}))


# ---------------------------------------------------------------------------
# The five gpt-oss-shaped workloads.  Seed = workload number.
# ---------------------------------------------------------------------------

def tiny_prefill_fp32(seed: int = 1) -> Workload:
    """fp32 causal prefill: 1 x 128 tokens, 4 query heads on 1 KV head, D=64, one KV block."""
    return make_workload("tiny_prefill_fp32_b1_s128_h4g4_d64", dtype="fp32", kind="prefill",
                         seqlens_q=[128], seqlens_k=[128], num_q_heads=4, num_kv_heads=1,
                         head_dim=64, seed=seed, causal=True)


def batched_decode(seed: int = 2, batch: int = 32, kv_len: int = 4096, num_chunks: int = 8) -> Workload:
    """bf16 decode: 32 sequences x 1 query token over 4096 cached keys, 64/8 heads, 8 KV chunks."""
    return make_workload(f"decode_bf16_b{batch}_kv{kv_len}_h64g8_d64_split{num_chunks}",
                         dtype="bf16", kind="decode", seqlens_q=[1] * batch,
                         seqlens_k=[kv_len] * batch, num_q_heads=64, num_kv_heads=8,
                         head_dim=64, seed=seed, causal=False,
                         kv_chunk=-(-kv_len // num_chunks))


def causal_prefill(seed: int = 3, batch: int = 4, seqlen: int = 4096) -> Workload:
    """bf16 causal prefill: 4 x 4096 tokens, 64/8 heads, D=64."""
    return make_workload(f"prefill_bf16_b{batch}_s{seqlen}_h64g8_d64", dtype="bf16",
                         kind="prefill", seqlens_q=[seqlen] * batch, seqlens_k=[seqlen] * batch,
                         num_q_heads=64, num_kv_heads=8, head_dim=64, seed=seed, causal=True)


def _ragged_lengths(rng, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi, size=batch, endpoint=True)


def ragged_decode_lengths(seed: int = 4, batch: int = 8, lo: int = 1024,
                          hi: int = 131072) -> np.ndarray:
    """The KV lengths of the long-context decode workload (its first draw from ``seed``)."""
    return _ragged_lengths(np.random.default_rng(seed), batch, lo, hi)


def ragged_decode(seed: int = 4, batch: int = 8, lo: int = 1024, hi: int = 131072,
                  chunk: int = 2048) -> Workload:
    """bf16 long-context decode: 8 sequences, KV length uniform in [1024, 131072], chunk 2048,
    sinks with standard deviation 2."""
    rng = np.random.default_rng(seed)
    lens = _ragged_lengths(rng, batch, lo, hi)
    return make_workload(f"ragged_decode_bf16_b{batch}_kv{lo}-{hi}_h64g8_d64_chunk{chunk}",
                         dtype="bf16", kind="decode", seqlens_q=[1] * batch,
                         seqlens_k=lens.tolist(), num_q_heads=64, num_kv_heads=8,
                         head_dim=64, seed=seed, causal=False, kv_chunk=chunk,
                         sink_sigma=2.0, rng=rng)


SINK_CATEGORIES = ("-inf", "-20", "0", "+20", "normal")


def mixed_varlen(seed: int = 5, n_prefill: int = 4, n_decode: int = 12, permute: bool = False) -> Workload:
    """bf16 packed batch: 4 prefill chunks (512-2048 new tokens over 0-8192 cached keys) and
    12 single-token decodes (1024-32768 keys); per-head sinks drawn from the categories
    {-inf, -20, 0, +20, N(0,1)}, every category present."""
    rng = np.random.default_rng(seed)
    new = rng.integers(512, 2048, size=n_prefill, endpoint=True)
    cached = rng.integers(0, 8192, size=n_prefill, endpoint=True)
    dec = rng.integers(1024, 32768, size=n_decode, endpoint=True)
    lq = [int(n) for n in new] + [1] * n_decode
    lk = [int(c + n) for c, n in zip(cached, new)] + [int(x) for x in dec]
    if permute:
        order = rng.permutation(len(lq))
        lq = [lq[i] for i in order]
        lk = [lk[i] for i in order]
    hq, hkv, d = 64, 8, 64
    cu_q, cu_k = _cu(lq), _cu(lk)
    q, k, v, q16, k16, v16 = _draw_qkv(rng, int(cu_q[-1]), int(cu_k[-1]), hq, hkv, d, "bf16")
    while True:
        cat = rng.integers(0, len(SINK_CATEGORIES), size=hq)
        if len(np.unique(cat)) == len(SINK_CATEGORIES):
            break
    normal = rng.standard_normal(hq, dtype=np.float32)
    table = np.array([-np.inf, -20.0, 0.0, 20.0, 0.0], dtype=np.float32)
    sinks = np.where(cat == 4, normal, table[cat]).astype(np.float32)
    name = "mixed_varlen_bf16_16seq_h64g8_d64" + ("_permuted" if permute else "")
    return Workload(name=name, dtype="bf16", kind="mixed", num_q_heads=hq, num_kv_heads=hkv,
                    head_dim=d, cu_q=cu_q, cu_k=cu_k, q32=q, k32=k, v32=v, sinks=sinks,
                    causal=True, kv_chunk=2048, q16=q16, k16=k16, v16=v16,
                    meta={"sink_category": cat.astype(np.int32)})


WORKLOADS = {
    1: tiny_prefill_fp32,
    2: batched_decode,
    3: causal_prefill,
    4: ragged_decode,
    5: mixed_varlen,
}


def workload(i: int, **kw) -> Workload:
    """Workload number ``i`` (1..5) with its default seed (= i)."""
    return WORKLOADS[i](**kw)


def random_case(seed: int, *, dtype="bf16", batch=2, hq=8, hkv=2, d=64, max_q=70,
                max_k=300, causal=True, decode=False, sink_sigma=1.0, sink_values=None) -> Workload:
    """Small random varlen case (for parity tests that must span several tiles and a tail)."""
    rng = np.random.default_rng(seed)
    if decode:
        lq = [1] * batch
        lk = rng.integers(1, max_k, size=batch, endpoint=True).tolist()
    else:
        lq = rng.integers(1, max_q, size=batch, endpoint=True).tolist()
        lk = [int(x) + int(rng.integers(0, max(1, max_k - max_q) + 1)) for x in lq]
    return make_workload(f"random_{seed}", dtype=dtype, kind="decode" if decode else "prefill",
                         seqlens_q=lq, seqlens_k=lk, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, seed=seed, causal=causal, sink_sigma=sink_sigma,
                         sink_values=sink_values, rng=rng)


def router_logits(seed: int, tokens: int, experts: int, ties: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Seeded router logits for the expert-routing step: bf16 bits [tokens, experts]
    (uint16) and their exact float32 values.  N(0, 1) draws rounded to bf16, or, with
    ``ties``, small integers in [-3, 3] (many equal logits) with some -0.0 entries."""
    rng = np.random.default_rng(seed)
    if ties:
        x = rng.integers(-3, 4, size=(tokens, experts)).astype(np.float32)
        x[rng.random((tokens, experts)) < 0.05] = -0.0
    else:
        x = rng.standard_normal((tokens, experts), dtype=np.float32)
    bits = bf16_round(x)
    return bits, bf16_widen(bits)


def yarn_table(rows: int, d: int = 64, *, theta: float = 150000.0, factor: float = 32.0,
               original_max: int = 4096, beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Rotary table [rows, d] float32 with YaRN frequency scaling (Peng et al., "YaRN:
    Efficient Context Window Extension of Large Language Models"): base frequencies
    theta^(-2i/d); a frequency whose wavelength fits r = original_max / wavelength
    times into the original context keeps its value when r > beta_fast, is divided by
    `factor` when r < beta_slow, and is blended linearly in between; cos and sin are
    multiplied by the attention scale 0.1 ln(factor) + 1.  Row p: cos(p w_i) for
    i < d/2, then sin(p w_i).  The parameter values are inputs of the workload (the
    pages name YaRN but give none)."""
    i = np.arange(d // 2, dtype=np.float64)
    base = theta ** (-2.0 * i / d)
    r = original_max * base / (2 * np.pi)
    keep = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    w = base * ((1.0 - keep) / factor + keep)
    scale = 0.1 * np.log(factor) + 1.0 if factor > 1.0 else 1.0
    ang = np.arange(rows, dtype=np.float64)[:, None] * w[None, :]
    return (np.concatenate([np.cos(ang), np.sin(ang)], axis=1) * scale).astype(np.float32)


def qkv_epilogue_inputs(seed: int, tokens: int, hq: int, hkv: int, d: int = 64,
                        max_pos: int = 8192):
    """Seeded inputs of the bias + rotary epilogue: qkv [tokens, (hq + 2 hkv) d] and
    bias [(hq + 2 hkv) d] as bf16 bits with their float32 values, positions [tokens]
    int32 (varlen: sequences of random length restarting at 0), and the YaRN table."""
    rng = np.random.default_rng(seed)
    width = (hq + 2 * hkv) * d
    qkv_bits = bf16_round(rng.standard_normal((tokens, width), dtype=np.float32))
    bias_bits = bf16_round(0.1 * rng.standard_normal(width, dtype=np.float32))
    pos = np.empty(tokens, dtype=np.int32)
    at = 0
    while at < tokens:
        n = int(rng.integers(1, min(max_pos, tokens) + 1))
        n = min(n, tokens - at)
        pos[at:at + n] = np.arange(n, dtype=np.int32)
        at += n
    return (qkv_bits, bf16_widen(qkv_bits), bias_bits, bf16_widen(bias_bits), pos,
            yarn_table(max_pos, d))
