"""GPU parity on seeded random shapes: the three attention reads (windowed ring with or without
slack, full context, verification) over random dtype, head_dim, KV heads, group size, batch,
lengths, sinks, window, slack, host bound and candidate count, each against the float64 oracle
(Windowed-MTP abstract: the windowed draft attends sinks plus a recent window, the native draft
and the verification attend the whole cache). The cases are fixed by their seeds, so a failure
names a reproducible shape."""
import math

import numpy as np
import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import (DEV, append_all, append_each, compare, logical_kv, ocode, oracle_kv,
                        run_full, run_verify, run_windowed, say, tdtype, tokens)

pytestmark = pytest.mark.gpu

N_CASES = 36


def _case(seed):
    r = np.random.default_rng(9000 + seed)
    c = {
        "kind": ("windowed", "full", "verify")[seed % 3],
        "dt": str(r.choice(["bf16", "f32"])),
        "d": int(r.choice([64, 128, 256])),
        "Hkv": int(r.choice([1, 2, 4])),
        "G": int(r.choice([1, 2, 4, 8, 16, 32])),
        "B": int(r.integers(1, 4)),
    }
    c["lens"] = [int(x) for x in r.integers(1, 3000, size=c["B"])]
    if c["kind"] == "windowed":
        c["S"] = int(r.integers(0, 9))
        c["W"] = int(r.choice([1, 7, 64, 300, 1000]))
        c["slack"] = int(r.choice([0, 0, 1, 3]))
    elif c["kind"] == "full":
        c["extra"] = int(r.integers(0, 2000))
    else:
        c["m"] = int(r.integers(1, 9))
        c["lens"] = [max(x, c["m"]) for x in c["lens"]]
        c["extra"] = int(r.integers(0, 500))
    return c


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    c = _case(seed)
    dt, d, Hkv, G, B, lens = c["dt"], c["d"], c["Hkv"], c["G"], c["B"], c["lens"]
    Hq = G * Hkv
    scale = 1.0 / math.sqrt(d)
    say(f"random case {seed}: {c}")
    K, V = logical_kv(900 + seed, B, Hkv, d, max(lens), tdtype(dt))
    kv = oracle_kv(K, V, dt)
    if c["kind"] == "windowed":
        ring = W.KVCache.ring(B, Hkv, d, c["S"], c["W"], tdtype(dt), slack=c["slack"])
        pre = [n - 1 for n in lens]
        append_each(ring, K, V, [0] * B, pre)
        append_all(ring, K, V, pre, 1)
        q = synth.queries(950 + seed, 0, B, 1, Hq, d, tdtype(dt), DEV)
        out, lse = run_windowed(ring, q, Hq, scale)
        ref_o, ref_l = oracle.draft_windowed(synth.host_array(q), ocode(dt), kv, lens, c["S"],
                                             c["W"], scale)
    else:
        m = c.get("m", 1)
        cap = max(lens) + c["extra"] + 1
        bound = max(lens) + (c["extra"] // 2)
        cache = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt))
        append_each(cache, K, V, [0] * B, lens)
        q = synth.queries(950 + seed, 0, B, m, Hq, d, tdtype(dt), DEV)
        if c["kind"] == "full":
            out, lse = run_full(cache, q, Hq, scale, bound)
            ref_o, ref_l = oracle.draft_full(synth.host_array(q), ocode(dt), kv, lens, scale)
        else:
            out, lse = run_verify(cache, q, Hq, scale, bound)
            ref_o, ref_l = oracle.verify(synth.host_array(q), ocode(dt), kv, lens, scale)
    compare(out, lse, ref_o, ref_l, dt, f"random {c['kind']} case {seed}")


N_STEP_CASES = 18


@pytest.mark.parametrize("seed", range(N_STEP_CASES))
def test_random_fused_step(seed):
    """The fused calls (append, then attend, in one call) on random shapes: the result covers the
    appended tokens, and the cache holds them afterwards (its length grew by their count)."""
    c = _case(100 + seed)
    dt, d, Hkv, G, B, lens = c["dt"], c["d"], c["Hkv"], c["G"], c["B"], c["lens"]
    Hq = G * Hkv
    scale = 1.0 / math.sqrt(d)
    m = c.get("m", 1)
    say(f"random fused step {seed}: {c}")
    K, V = logical_kv(700 + seed, B, Hkv, d, max(lens), tdtype(dt))
    kv = oracle_kv(K, V, dt)
    pre = [n - m for n in lens]  # the step appends the last m positions of every sequence
    kn = torch.stack([tokens(K, b, pre[b], lens[b]) for b in range(B)])
    vn = torch.stack([tokens(V, b, pre[b], lens[b]) for b in range(B)])
    q = synth.queries(750 + seed, 0, B, m, Hq, d, tdtype(dt), DEV)
    out = torch.full((B, m, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, m, Hq), float("nan"), dtype=torch.float32, device=DEV)
    if c["kind"] == "windowed":
        cache = W.KVCache.ring(B, Hkv, d, c["S"], c["W"], tdtype(dt), slack=c["slack"])
        append_each(cache, K, V, [0] * B, pre)
        ws = W.workspace(B, Hq, Hkv, d, 1, cache.capacity)
        W.wmtp_draft_step_windowed(cache, kn, vn, q, Hq, scale, out, lse, ws)
        ref_o, ref_l = oracle.draft_windowed(synth.host_array(q), ocode(dt), kv, lens, c["S"],
                                             c["W"], scale)
    else:
        cap = max(lens) + c["extra"] + 1
        bound = max(lens) + (c["extra"] // 2)
        cache = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt))
        append_each(cache, K, V, [0] * B, pre)
        ws = W.workspace(B, Hq, Hkv, d, m, bound)
        if c["kind"] == "full":
            W.wmtp_draft_step_full(cache, kn, vn, q, Hq, scale, bound, out, lse, ws)
            ref_o, ref_l = oracle.draft_full(synth.host_array(q), ocode(dt), kv, lens, scale)
        else:
            W.wmtp_verify_step(cache, kn, vn, q, m, Hq, scale, bound, out, lse, ws)
            ref_o, ref_l = oracle.verify(synth.host_array(q), ocode(dt), kv, lens, scale)
    compare(out, lse, ref_o, ref_l, dt, f"random fused {c['kind']} step {seed}")
    assert cache.seq_len.cpu().tolist() == lens
