"""The allocation-free windowed draft step (wmtp_draft_step_windowed_noalloc) against
wmtp_draft_step_windowed on identical rings, through the C ABI: outputs, lse, ring bytes, tags
and lengths equal bit for bit, on two calls in a row (the second on a smaller ring, so whatever
the first left in the shared static scratch must not leak into it)."""
import math

import pytest
import torch

from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import DEV, logical_kv, say, tdtype, tokens

pytestmark = pytest.mark.gpu


def _ring_pair(seed, B, Hkv, d, S, Wn, slack, n, dt):
    """Two rings holding the same n appended tokens, and the next token's rows."""
    K, V = logical_kv(seed, B, Hkv, d, n + 1, tdtype(dt))
    rings = []
    for _ in range(2):
        r = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=slack)
        kn = torch.stack([tokens(K, b, 0, n) for b in range(B)])
        vn = torch.stack([tokens(V, b, 0, n) for b in range(B)])
        W.wmtp_ring_append(r, kn, vn, n)
        rings.append(r)
    k1 = torch.stack([tokens(K, b, n, n + 1) for b in range(B)])
    v1 = torch.stack([tokens(V, b, n, n + 1) for b in range(B)])
    return rings, k1, v1


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_step_equals_the_workspace_step(dt):
    cases = [  # (B, Hkv, G, d, S, W, slack, n): the second call is smaller than the first
        (3, 2, 16, 256 if dt == "bf16" else 128, 4, 4096, 2, 9000),
        (1, 2, 4, 64, 4, 256, 0, 1000),
    ]
    for i, (B, Hkv, G, d, S, Wn, slack, n) in enumerate(cases):
        Hq = G * Hkv
        say(f"noalloc windowed step {dt} call {i}: B={B} Hq={Hq} Hkv={Hkv} d={d} S={S} W={Wn} "
            f"slack={slack} n={n}")
        (ra, rb), k1, v1 = _ring_pair(71 + i, B, Hkv, d, S, Wn, slack, n, dt)
        q = synth.queries(72 + i, 0, B, 1, Hq, d, tdtype(dt), DEV)
        scale = 1.0 / math.sqrt(d)
        outs = []
        for r, noalloc in ((ra, False), (rb, True)):
            out = torch.full((B, 1, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
            lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device=DEV)
            if noalloc:
                W.wmtp_draft_step_windowed_noalloc(r, k1, v1, q, Hq, scale, out, lse)
            else:
                W.wmtp_draft_step_windowed(r, k1, v1, q, Hq, scale, out, lse,
                                           W.workspace(B, Hq, Hkv, d, 1, r.capacity))
            outs.append((out, lse))
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0][0]).all(), "workspace step: non-finite output"
        assert torch.equal(outs[0][0], outs[1][0]), f"call {i}: outputs differ"
        assert torch.equal(outs[0][1], outs[1][1]), f"call {i}: lse differ"
        for name in ("k", "v", "pos", "seq_len"):
            assert torch.equal(getattr(ra, name), getattr(rb, name)), f"call {i}: ring {name} differs"


def test_noalloc_step_refuses_a_step_larger_than_its_scratch():
    """A step whose partials exceed WMTP_NOALLOC_SCRATCH_BYTES is refused before anything runs."""
    B, Hkv, Hq, d = 1024, 2, 32, 256  # 2048 (sequence, KV head) pairs: 32 MB of partials
    ring = W.KVCache.ring(B, Hkv, d, 4, 256, torch.bfloat16)
    q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros((B, 1, Hkv, d), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=DEV)
    assert W.lib().wmtp_attn_workspace_bytes(B, Hq, Hkv, d, 1, ring.capacity) > 16 << 20
    st = W.wmtp_draft_step_windowed_noalloc(ring, kn, kn, q, Hq, 0.1, out, None, check=False)
    assert st == W.WMTP_ERR_WORKSPACE
    assert int(ring.seq_len.sum().item()) == 0  # nothing ran
