"""The streaming-read yardstick (sink_attn_read_probe): its per-workgroup XOR digests
combine to the XOR of every 32-bit word of the buffer, for ragged sizes and any
number of workgroups, so the pass that bench.py times reads every byte once."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [
    (0, 3),
    (16, 1),
    (16 * 7919, 1),
    (16 * 7919, 5),
    (10 * (1 << 20) + 16 * 37, 1024),
    (64 << 20, 2048),
])
def test_read_probe_digest(nbytes, blocks):
    import torch
    import gqa_attention_head_amd as sa

    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = sa.read_probe(buf, num_blocks=blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) if blocks else 0
    want = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert int(got) == int(want)
