"""GPU parity on a cache too large for 32-bit byte offsets: 8.6 GB per K and V tensor, so the rows
of the last sequence start more than 2^32 bytes into each tensor. The full-context draft and the
verification read (key-split and cooperative kernels) are compared with the float64 oracle on the
last sequence's last KV head (every query head that reads it) and on a short first sequence."""
import math

import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import DEV, compare, ocode, oracle_kv, run_full, run_verify, say

pytestmark = pytest.mark.gpu

SEED = 91


def _fill(cache: W.KVCache, b: int, n: int, chunk: int = 1 << 17):
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        cache.k[b, :, c0:c1] = synth.sequence_rows(SEED, synth.K_ID, b, c0, c1, cache.n_kv_heads,
                                                   cache.head_dim, cache.k.dtype, DEV)
        cache.v[b, :, c0:c1] = synth.sequence_rows(SEED, synth.V_ID, b, c0, c1, cache.n_kv_heads,
                                                   cache.head_dim, cache.v.dtype, DEV)


def test_offsets_past_four_gib():
    B, Hkv, d, G = 2, 4, 256, 8
    Hq = G * Hkv
    lens = [1000, (1 << 21) + 3]
    cap = (1 << 21) + 16
    dt = torch.bfloat16
    row_bytes = d * 2
    assert (1 * Hkv + Hkv - 1) * cap * row_bytes > (1 << 32)  # the last head's rows start past 2^32
    say(f"large cache: {B}x{Hkv}x{cap}x{d} bf16 ({2 * B * Hkv * cap * row_bytes / 1e9:.1f} GB)")
    cache = W.KVCache.contiguous(B, Hkv, d, cap, dt)
    for b, n in enumerate(lens):
        _fill(cache, b, n)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32, device=DEV))
    scale = 1.0 / math.sqrt(d)
    h = Hkv - 1  # the last KV head of the last sequence, and the query heads that read it
    heads = list(range(h * G, (h + 1) * G))
    say("large cache: host copies of the sampled rows")
    kv_last = oracle_kv(cache.k[1:2, h:h + 1, :lens[1]], cache.v[1:2, h:h + 1, :lens[1]], "bf16")
    kv_first = oracle_kv(cache.k[0:1, :, :lens[0]], cache.v[0:1, :, :lens[0]], "bf16")

    # draft step (key-split), verify with 16 and 32 rows (key-split: one and two row blocks) and
    # 48 (cooperative: more than the key-split kernel's 32 rows at head_dim 256)
    for m in (1, 2, 4, 6):
        q = synth.queries(SEED, m, B, m, Hq, d, dt, DEV)
        say(f"large cache: m={m} on the GPU")
        if m == 1:
            out, lse = run_full(cache, q, Hq, scale, cap)
            ref = lambda qh, kv, n: oracle.draft_full(qh, ocode("bf16"), kv, n, scale)
        else:
            out, lse = run_verify(cache, q, Hq, scale, cap)
            ref = lambda qh, kv, n: oracle.verify(qh, ocode("bf16"), kv, n, scale)
        say(f"large cache: m={m} oracle")
        qh = synth.host_array(q)
        r1, l1 = ref(qh[1:2, :, heads], kv_last, [lens[1]])
        compare(out[1:2, :, heads], lse[1:2, :, heads], r1, l1, "bf16",
                f"m={m}, last sequence, KV head {h}")
        r0, l0 = ref(qh[0:1], kv_first, [lens[0]])
        compare(out[0:1], lse[0:1], r0, l0, "bf16", f"m={m}, first sequence")

    # appends past 2^32 bytes: the plain append, then the one-call full-context draft step; the
    # rows land at positions lens[b] and lens[b] + 1 bit for bit, and the step's outputs equal
    # append-then-attend
    say("large cache: appends")
    toks = [synth.token_rows(SEED, synth.K_ID, b, lens[b], lens[b] + 2, Hkv, d, dt, DEV)
            for b in range(B)]
    vals = [synth.token_rows(SEED, synth.V_ID, b, lens[b], lens[b] + 2, Hkv, d, dt, DEV)
            for b in range(B)]
    kn = lambda i: torch.stack([t[i:i + 1] for t in toks]).contiguous()  # [B][1][Hkv][d]
    vn = lambda i: torch.stack([t[i:i + 1] for t in vals]).contiguous()
    W.wmtp_ring_append(cache, kn(0), vn(0), 1)
    q = synth.queries(SEED, 7, B, 1, Hq, d, dt, DEV)
    view = W.KVCache(cache.k, cache.v, None, cache.seq_len.clone(), B, Hkv, d, cap, cap, 0,
                     cache.dtype)
    W.wmtp_ring_append(cache, kn(1), vn(1), 1)
    o1, l1 = run_full(cache, q, Hq, scale, cap)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    W.wmtp_draft_step_full(view, kn(1), vn(1), q, Hq, scale, cap, o2, l2,
                           W.workspace(B, Hq, Hkv, d, 1, cap))
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "one-call step differs past 2^32 bytes"
    for b in range(B):
        for i in range(2):
            assert torch.equal(cache.k[b, :, lens[b] + i], toks[b][i]), f"K row {b}/{i}"
            assert torch.equal(cache.v[b, :, lens[b] + i], vals[b][i]), f"V row {b}/{i}"
    assert cache.seq_len.tolist() == [n + 2 for n in lens]
    assert view.seq_len.tolist() == [n + 2 for n in lens]
