"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark times.

Every output the oracle can afford is compared (all heads of every draft step at 1M context take a
few seconds of float64 on the host); the batched 10,000-step ring run is compared at sampled steps
(first, last, every 500th, and every step at which a sequence's window wraps back onto its first
window slot), with the ring's bytes and position tags checked bit for bit at the same steps.

The benchmark times the one-call steps (wmtp_draft_step_windowed / _full, wmtp_verify_step). At the
million-token sizes they run beside the separate calls on the same bytes and must equal them bit for
bit (outputs, lse, cache rows, tags, lengths), so the oracle comparison covers them too.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import configs, synth
from gpu_common import (DEV, TOL, append_all, append_each, compare, ocode, oracle_kv, run_full,
                        run_verify, run_windowed, say, tdtype, tokens)

pytestmark = pytest.mark.gpu


def fill_prefix(cache: W.KVCache, seed: int, length: int, dt, k_scale=None, chunk=1 << 17):
    """Set-up only: write positions [0, length) of every sequence straight into a contiguous cache
    (the same rows an append of them would copy) and set seq_len."""
    for b in range(cache.batch):
        for c0 in range(0, length, chunk):
            c1 = min(length, c0 + chunk)
            cache.k[b, :, c0:c1] = synth.sequence_rows(seed, synth.K_ID, b, c0, c1, cache.n_kv_heads,
                                                       cache.head_dim, dt, DEV, k_scale)
            cache.v[b, :, c0:c1] = synth.sequence_rows(seed, synth.V_ID, b, c0, c1, cache.n_kv_heads,
                                                       cache.head_dim, dt, DEV)
    cache.seq_len.fill_(length)


def kv_of(cache: W.KVCache, n: int, dtname: str) -> oracle.LogicalKV:
    return oracle_kv(cache.k[:, :, :n], cache.v[:, :, :n], dtname)


def draft_steps(wl, k_scale=None, full_heads=None, fused=False):
    """The draft loop of one workload: k steps, each appending its token to the ring and to the
    contiguous cache, then attending (windowed and full) with that step's query. With `fused`, the
    one-call steps run beside them on a copy of the ring and on the same contiguous rows (own
    length counter) and must give the same bits."""
    dt = tdtype(wl.dtype)
    L, k, d = wl.context, wl.draft_depth, wl.head_dim
    scale = 1.0 / math.sqrt(d)
    say(f"{wl.name}: prefix of {L} tokens")
    cache = W.KVCache.contiguous(1, wl.n_kv_heads, d, L + k, dt)
    fill_prefix(cache, wl.seed, L + k, dt, k_scale)  # rows of the draft tokens too (oracle input)
    kv = kv_of(cache, L + k, wl.dtype)  # the generator's bytes, before any kernel touches them
    cache.seq_len.fill_(L)
    ring = W.KVCache.ring(1, wl.n_kv_heads, d, wl.sink, wl.window, dt)
    # the prefix goes through one bulk append (survivor-only writes)
    append_each(ring, cache.k, cache.v, [0], [L])
    model = oracle.RingModel(1, wl.sink, wl.window)
    model.append(0, L)
    if fused:
        ring2 = W.KVCache(ring.k.clone(), ring.v.clone(), ring.pos.clone(), ring.seq_len.clone(),
                          1, ring.n_kv_heads, d, ring.capacity, ring.sink, ring.window, ring.dtype)
        view2 = W.KVCache(cache.k, cache.v, None, cache.seq_len.clone(), 1, cache.n_kv_heads, d,
                          cache.capacity, cache.capacity, 0, cache.dtype)
        ws_win = W.workspace(1, wl.n_q_heads, ring.n_kv_heads, d, 1, ring.capacity)
        ws_full = W.workspace(1, wl.n_q_heads, cache.n_kv_heads, d, 1, L + k)
        out2 = torch.empty((1, 1, wl.n_q_heads, d), dtype=torch.float32, device=DEV)
        lse2 = torch.empty((1, 1, wl.n_q_heads), dtype=torch.float32, device=DEV)
    worst = 0.0
    for i in range(k):
        n = L + i + 1
        say(f"{wl.name}: draft step {i} (n={n})")
        append_all(ring, cache.k, cache.v, [n - 1], 1)
        append_all(cache, cache.k, cache.v, [n - 1], 1)
        model.append(0, 1)
        q = synth.queries(wl.seed, i, 1, 1, wl.n_q_heads, d, dt, DEV)
        ow, lw = run_windowed(ring, q, wl.n_q_heads, scale)
        of, lf = run_full(cache, q, wl.n_q_heads, scale, L + k)
        qh = synth.host_array(q)
        rw, rlw = oracle.draft_windowed(qh, ocode(wl.dtype), kv, [n], wl.sink, wl.window, scale)
        worst = max(worst, compare(ow, lw, rw, rlw, wl.dtype, f"windowed step {i}")[0])
        heads = list(range(wl.n_q_heads)) if full_heads is None else full_heads(i)
        rf, rlf = oracle.draft_full(qh[:, :, heads], ocode(wl.dtype),
                                    _head_subset(kv, heads, wl), [n], scale)
        worst = max(worst, compare(of[:, :, heads], lf[:, :, heads], rf, rlf, wl.dtype,
                                   f"full step {i} ({len(heads)} heads)")[0])
        if fused:
            kn = tokens(cache.k, 0, n - 1, n)[None]
            vn = tokens(cache.v, 0, n - 1, n)[None]
            W.wmtp_draft_step_windowed(ring2, kn, vn, q, wl.n_q_heads, scale, out2, lse2, ws_win)
            assert torch.equal(out2, ow) and torch.equal(lse2, lw), f"fused windowed step {i}"
            W.wmtp_draft_step_full(view2, kn, vn, q, wl.n_q_heads, scale, L + k, out2, lse2,
                                   ws_full)
            assert torch.equal(out2, of) and torch.equal(lse2, lf), f"fused full step {i}"
            assert torch.equal(view2.seq_len, cache.seq_len), f"fused full step {i}: length"
            say(f"  fused steps {i}: equal to append-then-attend bit for bit")
    if fused:
        for a, b_ in ((ring2.k, ring.k), (ring2.v, ring.v), (ring2.pos, ring.pos),
                      (ring2.seq_len, ring.seq_len)):
            assert torch.equal(a, b_), "fused windowed steps: ring state differs"
    # the ring holds exactly the sinks and the last W positions, bit for bit
    tags = ring.pos.cpu().numpy().astype(np.int64)
    assert np.array_equal(tags, model.tags)
    rk, rv = oracle.ring_expected(model, kv)
    occ = model.occupied_slots(0)
    assert np.array_equal(synth.host_array(ring.k)[0][:, occ], rk[0][:, occ])
    assert np.array_equal(synth.host_array(ring.v)[0][:, occ], rv[0][:, occ])
    return worst


def _head_subset(kv: oracle.LogicalKV, heads, wl):
    """The oracle maps query head hq to KV head hq // G; a subset of query heads keeps that map by
    repeating their KV heads."""
    G = wl.n_q_heads // wl.n_kv_heads
    if len(heads) == wl.n_q_heads:
        return kv
    kvh = [h // G for h in heads]
    return oracle.LogicalKV(kv.k[:, kvh], kv.v[:, kvh], kv.dtype, kv.segments)


def test_tiny_draft_fp32():
    wl = configs.TINY
    draft_steps(wl)


def test_tiny_window_covers_all_equivalence():
    """S + W >= n: windowed attention is full attention (the tiny workload at L = 256)."""
    wl = configs.TINY
    dt = tdtype(wl.dtype)
    L, d = 256, wl.head_dim
    say("tiny workload at L=256: windowed == full")
    cache = W.KVCache.contiguous(1, wl.n_kv_heads, d, L + 1, dt)
    fill_prefix(cache, wl.seed, L + 1, dt)
    cache.seq_len.fill_(L)
    kv = kv_of(cache, L + 1, wl.dtype)
    ring = W.KVCache.ring(1, wl.n_kv_heads, d, wl.sink, wl.window, dt)
    append_each(ring, cache.k, cache.v, [0], [L + 1])
    append_all(cache, cache.k, cache.v, [L], 1)
    q = synth.queries(wl.seed, 0, 1, 1, wl.n_q_heads, d, dt, DEV)
    scale = 1.0 / math.sqrt(d)
    ow, lw = run_windowed(ring, q, wl.n_q_heads, scale)
    of, lf = run_full(cache, q, wl.n_q_heads, scale, L + 1)
    qh = synth.host_array(q)
    rw, rlw = oracle.draft_windowed(qh, ocode(wl.dtype), kv, [L + 1], wl.sink, wl.window, scale)
    rf, rlf = oracle.draft_full(qh, ocode(wl.dtype), kv, [L + 1], scale)
    assert np.array_equal(rw, rf) and np.array_equal(rlw, rlf)  # the oracle: identical sets
    compare(ow, lw, rf, rlf, wl.dtype, "windowed vs full oracle")
    compare(of, lf, rf, rlf, wl.dtype, "full vs full oracle")


def test_mid_context_three_steps():
    wl = configs.MID
    draft_steps(wl, k_scale=wl.k_scale, fused=True)


def test_million_token_five_steps():
    wl = configs.MILLION
    draft_steps(wl, fused=True)


def test_verify_million_tokens():
    wl = configs.VERIFY
    dt = tdtype(wl.dtype)
    L, m, d = wl.context, wl.verify_m, wl.head_dim
    scale = 1.0 / math.sqrt(d)
    say(f"{wl.name}: prefix {L}, {m} candidates")
    cache = W.KVCache.contiguous(1, wl.n_kv_heads, d, L + m, dt)
    fill_prefix(cache, wl.seed, L + m, dt)
    kv = kv_of(cache, L + m, wl.dtype)  # the generator's bytes, before any kernel touches them
    cache.seq_len.fill_(L)
    view2 = W.KVCache(cache.k, cache.v, None, cache.seq_len.clone(), 1, cache.n_kv_heads, d,
                      cache.capacity, cache.capacity, 0, cache.dtype)
    append_all(cache, cache.k, cache.v, [L], m)  # the candidates, through the append path
    q = synth.queries(wl.seed, 0, 1, m, wl.n_q_heads, d, dt, DEV)
    out, lse = run_verify(cache, q, wl.n_q_heads, scale, L + m)
    # the one-call verification step the benchmark times (append of the m candidates fused in),
    # on the same rows with its own length counter: the same bits
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    ws = W.workspace(1, wl.n_q_heads, wl.n_kv_heads, d, m, L + m)
    W.wmtp_verify_step(view2, tokens(cache.k, 0, L, L + m)[None], tokens(cache.v, 0, L, L + m)[None],
                       q, m, wl.n_q_heads, scale, L + m, out2, lse2, ws)
    assert torch.equal(out2, out) and torch.equal(lse2, lse), "fused verification step"
    assert torch.equal(view2.seq_len, cache.seq_len), "fused verification step: length"
    ref, rl = oracle.verify(synth.host_array(q), ocode(wl.dtype), kv, [L + m], scale)
    compare(out, lse, ref, rl, wl.dtype, "verify at 1M")
    # the causal rows differ from one another only through the candidates they see
    assert not torch.equal(out[:, 0], out[:, m - 1])


def test_batched_ring_10000_decode_steps():
    wl = configs.BATCHED
    dt = tdtype(wl.dtype)
    B, S, Wn, d, Hq, Hkv = wl.batch, wl.sink, wl.window, wl.head_dim, wl.n_q_heads, wl.n_kv_heads
    steps = wl.decode_steps * wl.draft_depth  # all drafts accepted: one token per draft step
    lens = [synth.uniform_int(wl.seed, synth.LEN_ID, b, wl.ragged_lo, wl.context) for b in range(B)]
    say(f"{wl.name}: lengths {lens}, {steps} draft steps")
    scale = 1.0 / math.sqrt(d)
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, dt)
    # rows the run touches: sinks, the last window of the prefix, and every appended token
    span = Wn + steps
    Ks = torch.stack([torch.cat([synth.sequence_rows(wl.seed, synth.K_ID, b, 0, S, Hkv, d, dt, DEV),
                                 synth.sequence_rows(wl.seed, synth.K_ID, b, lens[b] - Wn,
                                                     lens[b] + steps, Hkv, d, dt, DEV)], dim=1)
                      for b in range(B)])
    Vs = torch.stack([torch.cat([synth.sequence_rows(wl.seed, synth.V_ID, b, 0, S, Hkv, d, dt, DEV),
                                 synth.sequence_rows(wl.seed, synth.V_ID, b, lens[b] - Wn,
                                                     lens[b] + steps, Hkv, d, dt, DEV)], dim=1)
                      for b in range(B)])
    tok = lambda X, r0, r1: X[:, :, r0:r1].permute(0, 2, 1, 3).contiguous()
    # set-up: the ring state after L_b appends holds the sinks and positions L_b-W .. L_b-1
    W.wmtp_ring_append(ring, tok(Ks, 0, S), tok(Vs, 0, S), S)
    ring.seq_len.copy_(torch.tensor([n - Wn for n in lens], dtype=torch.int32, device=DEV))
    W.wmtp_ring_append(ring, tok(Ks, S, S + Wn), tok(Vs, S, S + Wn), Wn)
    kv = oracle.LogicalKV(synth.host_array(Ks), synth.host_array(Vs), ocode(wl.dtype),
                          [[(0, 0, S), (lens[b] - Wn, S, span)] for b in range(B)])
    # sampled steps: first, last, every 500th, and for each sequence every step whose token wraps
    # onto window slot S (its position p has (p - S) % W == 0)
    sample = {0, 1, steps - 1} | set(range(0, steps, 500))
    for b in range(B):
        sample |= set(range((S - lens[b]) % Wn, steps, Wn))
    say(f"{len(sample)} sampled steps")
    # host ring model of every append so far, advanced to each sampled step
    model = oracle.RingModel(B, S, Wn)
    for b in range(B):
        model.append(b, lens[b])
    in_model = 0  # draft steps the model has appended
    ws = W.workspace(B, Hq, Hkv, d, 1, S + Wn)
    out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)
    chunk = 4000
    worst = 0.0
    for c0 in range(0, steps, chunk):
        c1 = min(steps, c0 + chunk)
        # queries of steps c0..c1-1 (the counters synth.queries uses for m = 1), in one go
        pos = torch.arange(c0, c1, dtype=torch.int64, device=DEV)
        qs = torch.stack([synth.cast(synth.normal_rows(wl.seed, synth.Q_ID, b, pos, Hq, d, DEV), dt)
                          for b in range(B)], dim=1).unsqueeze(2)  # [steps][B][1][Hq][d]
        for i in range(c0, c1):
            r = S + Wn + i  # row of this step's token in Ks/Vs
            W.wmtp_ring_append(ring, tok(Ks, r, r + 1), tok(Vs, r, r + 1), 1)
            W.wmtp_draft_attn_windowed(ring, qs[i - c0], Hq, scale, out, lse, ws)
            if i not in sample:
                continue
            n = [lens[b] + i + 1 for b in range(B)]
            ref, rl = oracle.draft_windowed(synth.host_array(qs[i - c0]), ocode(wl.dtype), kv, n,
                                            S, Wn, scale)
            worst = max(worst, compare(out, lse, ref, rl, wl.dtype, f"batched step {i}")[0])
            for b in range(B):
                model.append(b, i + 1 - in_model)
            in_model = i + 1
            assert np.array_equal(model.n, n)
            assert np.array_equal(ring.pos.cpu().numpy().astype(np.int64), model.tags), f"tags {i}"
            rk, rv = oracle.ring_expected(model, kv)
            hk, hv = synth.host_array(ring.k), synth.host_array(ring.v)
            for b in range(B):
                occ = model.occupied_slots(b)
                assert np.array_equal(hk[b][:, occ], rk[b][:, occ]), f"K bytes, step {i}"
                assert np.array_equal(hv[b][:, occ], rv[b][:, occ]), f"V bytes, step {i}"
    assert int(ring.seq_len.cpu()[0]) == lens[0] + steps
    say(f"batched: worst max|out-ref| over sampled steps = {worst:.3e}")
