"""GPU parity of the MASW-style draft step (MASW page, section 4.1): the draft attends the sinks,
the exact local window of its ring and every memory slot materialised so far (slot K/V rows are
synthetic inputs, one per r raw tokens), through one call whose two reads share one log-sum-exp
merge. Compared with the float64 oracle over the union; slots discarded after a rejection
(section 4.3) no longer count."""
import math

import numpy as np
import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import DEV, append_each, compare, logical_kv, ocode, say, tdtype

pytestmark = pytest.mark.gpu

SLOT_K_ID, SLOT_V_ID = 11, 12  # generator streams of the synthetic memory-slot rows


def _slots(seed, B, Hkv, d, count, dt):
    k = torch.stack([synth.sequence_rows(seed, SLOT_K_ID, b, 0, count, Hkv, d, tdtype(dt), DEV)
                     for b in range(B)])
    v = torch.stack([synth.sequence_rows(seed, SLOT_V_ID, b, 0, count, Hkv, d, tdtype(dt), DEV)
                     for b in range(B)])
    return k, v  # [B][Hkv][count][d]


def _run(ring, slots, q, Hq, scale, max_slots):
    B, d = ring.batch, ring.head_dim
    out = torch.full((B, 1, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = W.masw_workspace(B, Hq, ring.n_kv_heads, d, ring.capacity, max_slots)
    W.wmtp_draft_attn_masw(ring, slots, q, Hq, scale, max_slots, out, lse, ws)
    return out, lse


@pytest.mark.parametrize("dt,d,G,r,lens,slack", [
    ("bf16", 128, 8, 8, [3000, 40], 0),
    ("bf16", 256, 16, 4, [1500], 3),
    ("bf16", 64, 4, 64, [5000, 700, 9], 0),
    ("bf16", 128, 32, 16, [2600], 2),      # 32 rows per KV head: cooperative kernel
    ("f32", 64, 8, 8, [1200, 260], 0),
    ("f32", 128, 4, 1, [333], 4),          # a slot per token
])
def test_masw_parity(dt, d, G, r, lens, slack):
    B, Hkv, S, Wn = len(lens), 2, 4, 128
    Hq = G * Hkv
    say(f"masw {dt} d={d} G={G} r={r} lens={lens} slack={slack}")
    K, V = logical_kv(61, B, Hkv, d, max(lens), tdtype(dt))
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=slack)
    append_each(ring, K, V, [0] * B, lens)
    n_slots = [n // r for n in lens]  # one slot per completed r-token block
    max_slots = max(max(n_slots), 1)
    sk, sv = _slots(62, B, Hkv, d, max_slots, dt)
    slots = W.KVCache.contiguous(B, Hkv, d, max_slots + 5, tdtype(dt))
    for b in range(B):  # the slots each sequence has materialised
        if n_slots[b]:
            sub = W.KVCache(slots.k[b:b + 1], slots.v[b:b + 1], None, slots.seq_len[b:b + 1], 1,
                            Hkv, d, slots.capacity, slots.capacity, 0, slots.dtype)
            W.wmtp_ring_append(sub, sk[b:b + 1, :, :n_slots[b]].permute(0, 2, 1, 3).contiguous(),
                               sv[b:b + 1, :, :n_slots[b]].permute(0, 2, 1, 3).contiguous(),
                               n_slots[b])
    q = synth.queries(63, 0, B, 1, Hq, d, tdtype(dt), DEV)
    scale = 1.0 / math.sqrt(d)
    out, lse = _run(ring, slots, q, Hq, scale, max_slots + 5)
    kv = oracle.contiguous_kv(synth.host_array(K), synth.host_array(V), ocode(dt))
    ro, rl = oracle.draft_masw(synth.host_array(q), ocode(dt), kv, lens, S, Wn,
                               synth.host_array(sk), synth.host_array(sv), n_slots, scale)
    compare(out, lse, ro, rl, dt, "masw")


def test_masw_without_slots_equals_windowed():
    dt, d, G, B, Hkv, S, Wn = "bf16", 128, 8, 2, 2, 4, 64
    Hq = G * Hkv
    say("masw with an empty slot memory == windowed")
    K, V = logical_kv(71, B, Hkv, d, 900, tdtype(dt))
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt))
    append_each(ring, K, V, [0] * B, [900, 500])
    slots = W.KVCache.contiguous(B, Hkv, d, 16, tdtype(dt))
    q = synth.queries(72, 0, B, 1, Hq, d, tdtype(dt), DEV)
    om, lm = _run(ring, slots, q, Hq, 0.1, 16)
    ow = torch.empty_like(om)
    lw = torch.empty_like(lm)
    W.wmtp_draft_attn_windowed(ring, q, Hq, 0.1, ow, lw, W.workspace(B, Hq, Hkv, d, 1, ring.capacity))
    assert torch.max(torch.abs(om - ow)).item() <= 2e-6
    assert torch.max(torch.abs(lm - lw)).item() <= 2e-6


def test_masw_slot_rollback_after_rejection():
    """Drafts that crossed an r-token boundary materialised a slot; after the rejection both the
    raw draft tokens and that slot are discarded (MASW page, section 4.3)."""
    dt, d, G, B, Hkv, S, Wn, r, k = "bf16", 128, 4, 1, 2, 4, 32, 4, 4
    Hq = G * Hkv
    say("masw rollback of raw tokens and slots")
    n0 = 202  # 50 slots; drafts 202..205 complete block 50 (positions 200..203) -> slot 50
    K, V = logical_kv(81, B, Hkv, d, n0 + k, tdtype(dt))
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=k)
    append_each(ring, K, V, [0], [n0 + k])
    sk, sv = _slots(82, B, Hkv, d, 51, dt)
    slots = W.KVCache.contiguous(B, Hkv, d, 64, tdtype(dt))
    W.wmtp_ring_append(slots, sk.permute(0, 2, 1, 3).contiguous(),
                       sv.permute(0, 2, 1, 3).contiguous(), 51)
    accepted = 1  # keep draft 202 only: n = 203, slots = 203 // 4 = 50
    W.wmtp_ring_rollback(ring, torch.tensor([k - accepted], dtype=torch.int32, device=DEV))
    W.wmtp_ring_rollback(slots, torch.tensor([51 - (n0 + accepted) // r], dtype=torch.int32,
                                             device=DEV))
    assert ring.seq_len.item() == n0 + accepted and slots.seq_len.item() == 50
    q = synth.queries(83, 0, B, 1, Hq, d, tdtype(dt), DEV)
    out, lse = _run(ring, slots, q, Hq, 0.125, 64)
    kv = oracle.contiguous_kv(synth.host_array(K), synth.host_array(V), ocode(dt))
    ro, rl = oracle.draft_masw(synth.host_array(q), ocode(dt), kv, [n0 + accepted], S, Wn,
                               synth.host_array(sk), synth.host_array(sv), [50], 0.125)
    compare(out, lse, ro, rl, dt, "masw after rollback")


@pytest.mark.parametrize("r", [64, 8])
def test_masw_million_token_context(r):
    """The benchmark's MASW step at its size and launch configuration: the million-token draft
    shapes (32 query / 2 KV heads, d 256, bf16, S 4, W 4096) at n = 1,048,577 with one memory slot
    per r raw tokens (16,384 or 131,072 slots), every query head against the oracle."""
    from draft_attention_amd import configs

    wl = configs.MILLION
    Hq, Hkv, d, S, Wn = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.sink, wl.window
    dt = torch.bfloat16
    n = wl.context + 1
    m = n // r
    say(f"masw at n={n}, r={r}: {m} slots")
    # the ring after n appends holds the sinks and the last W positions: append those only
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, dt)
    Ks = torch.cat([synth.sequence_rows(wl.seed, synth.K_ID, 0, 0, S, Hkv, d, dt, DEV),
                    synth.sequence_rows(wl.seed, synth.K_ID, 0, n - Wn, n, Hkv, d, dt, DEV)], dim=1)
    Vs = torch.cat([synth.sequence_rows(wl.seed, synth.V_ID, 0, 0, S, Hkv, d, dt, DEV),
                    synth.sequence_rows(wl.seed, synth.V_ID, 0, n - Wn, n, Hkv, d, dt, DEV)], dim=1)
    tok = lambda X, r0, r1: X[:, r0:r1].permute(1, 0, 2).contiguous()[None]
    W.wmtp_ring_append(ring, tok(Ks, 0, S), tok(Vs, 0, S), S)
    ring.seq_len.fill_(n - Wn)
    W.wmtp_ring_append(ring, tok(Ks, S, S + Wn), tok(Vs, S, S + Wn), Wn)
    sk, sv = _slots(wl.seed + 3, 1, Hkv, d, m, "bf16")
    slots = W.KVCache.contiguous(1, Hkv, d, m, dt)
    for c0 in range(0, m, 1 << 16):
        c1 = min(m, c0 + (1 << 16))
        W.wmtp_ring_append(slots, sk[:, :, c0:c1].permute(0, 2, 1, 3).contiguous(),
                           sv[:, :, c0:c1].permute(0, 2, 1, 3).contiguous(), c1 - c0)
    q = synth.queries(wl.seed + 2, 0, 1, 1, Hq, d, dt, DEV)
    scale = 1.0 / math.sqrt(d)
    out, lse = _run(ring, slots, q, Hq, scale, m)
    kv = oracle.LogicalKV(synth.host_array(Ks)[None], synth.host_array(Vs)[None], oracle.BF16,
                          [[(0, 0, S), (n - Wn, S, Wn)]])
    ro, rl = oracle.draft_masw(synth.host_array(q), oracle.BF16, kv, [n], S, Wn,
                               synth.host_array(sk), synth.host_array(sv), [m], scale)
    compare(out, lse, ro, rl, "bf16", f"masw at 1M, r={r}")
