"""GPU parity of the speculative-decoding steps around the draft attention: rings with slack
slots, rollback of rejected draft tokens, windowed attention after rollbacks, and greedy
acceptance from the target's logits. Ring tags, lengths and bytes must match the host model bit
for bit; acceptance outputs are integers and must match the oracle exactly; attention matches the
float64 oracle within the usual tolerances."""
import math

import numpy as np
import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import DEV, append_each, compare, logical_kv, ocode, say, tdtype

pytestmark = pytest.mark.gpu


def _check_ring(ring: W.KVCache, model: oracle.RingModel, seq_k, seq_v, what: str):
    """Tags and lengths equal the model's; every occupied slot holds the bytes of the position
    its tag names (seq_k/seq_v: host arrays [B][Hkv][positions][d] of the final content)."""
    tags = ring.pos.cpu().numpy().astype(np.int64)
    assert np.array_equal(tags, model.tags), f"{what}: position tags differ"
    assert np.array_equal(ring.seq_len.cpu().numpy().astype(np.int64), model.n), f"{what}: seq_len"
    hk, hv = synth.host_array(ring.k), synth.host_array(ring.v)
    for b in range(ring.batch):
        if ring.window >= 1:
            model.attended_slots(b)  # raises if the model lost a position the window needs
        occ = model.occupied_slots(b)
        pos = model.tags[b, occ]
        assert np.array_equal(hk[b][:, occ], seq_k[b][:, pos]), f"{what}: K bytes of sequence {b}"
        assert np.array_equal(hv[b][:, occ], seq_v[b][:, pos]), f"{what}: V bytes of sequence {b}"


class _Spec:
    """Device ring + host model + the final content of every position of every sequence. Draft
    tokens of round r get their own seeded rows, so a position rewritten after a rollback holds
    different bytes from the rejected token it replaces."""

    def __init__(self, B, Hkv, d, S, Wn, slack, dt, seed):
        self.B, self.Hkv, self.d, self.dt, self.seed = B, Hkv, d, dt, seed
        self.ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=slack)
        self.model = oracle.RingModel(B, S, Wn, slack)
        self.seq_k = [np.zeros((Hkv, 0, d), dtype=self._np()) for _ in range(B)]
        self.seq_v = [np.zeros((Hkv, 0, d), dtype=self._np()) for _ in range(B)]
        self.round = 0

    def _np(self):
        return np.uint16 if self.dt == "bf16" else np.float32

    def append(self, t: int):
        """Append t tokens to every sequence in one call."""
        self.round += 1
        rows_k, rows_v = [], []
        for b in range(self.B):
            n = int(self.model.n[b])
            sd = self.seed + 7919 * self.round
            rows_k.append(synth.token_rows(sd, synth.KNEW_ID, b, n, n + t, self.Hkv, self.d,
                                           tdtype(self.dt), DEV))
            rows_v.append(synth.token_rows(sd, synth.VNEW_ID, b, n, n + t, self.Hkv, self.d,
                                           tdtype(self.dt), DEV))
        kn, vn = torch.stack(rows_k), torch.stack(rows_v)
        W.wmtp_ring_append(self.ring, kn, vn, t)
        hk, hv = synth.host_array(kn), synth.host_array(vn)  # [B][t][Hkv][d]
        for b in range(self.B):
            n = int(self.model.n[b])
            keep = n  # positions >= n are replaced
            self.seq_k[b] = np.concatenate([self.seq_k[b][:, :keep], hk[b].transpose(1, 0, 2)], 1)
            self.seq_v[b] = np.concatenate([self.seq_v[b][:, :keep], hv[b].transpose(1, 0, 2)], 1)
            self.model.append(b, t)

    def rollback(self, drops):
        W.wmtp_ring_rollback(self.ring, torch.tensor(drops, dtype=torch.int32, device=DEV))
        for b, d in enumerate(drops):
            self.model.rollback(b, int(d))  # the depth the device must have taken
            n = int(self.model.n[b])
            self.seq_k[b] = self.seq_k[b][:, :n]
            self.seq_v[b] = self.seq_v[b][:, :n]

    def logical_kv(self):
        n_max = max(int(x) for x in self.model.n)
        k = np.zeros((self.B, self.Hkv, n_max, self.d), dtype=self._np())
        v = np.zeros_like(k)
        for b in range(self.B):
            k[b, :, :self.seq_k[b].shape[1]] = self.seq_k[b]
            v[b, :, :self.seq_v[b].shape[1]] = self.seq_v[b]
        return oracle.contiguous_kv(k, v, ocode(self.dt))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("S,Wn,slack", [(4, 16, 5), (0, 7, 3), (3, 1, 2), (4, 64, 6)])
def test_append_and_rollback_bitexact(dt, S, Wn, slack):
    B, Hkv, d = 3, 2, 128
    say(f"ring slack append/rollback {dt} S={S} W={Wn} slack={slack}")
    spec = _Spec(B, Hkv, d, S, Wn, slack, dt, seed=31)
    rng = np.random.default_rng(S * 1000 + Wn * 10 + slack)
    spec.append(S + Wn + slack + 9)  # prefill past one wrap
    _check_ring(spec.ring, spec.model, spec.seq_k, spec.seq_v, "after prefill")
    for step in range(12):
        t = int(rng.integers(1, slack + 2))
        spec.append(t)
        drops = rng.integers(-1, slack + 3, size=B).tolist()  # includes clamped and negative
        spec.rollback(drops)
        _check_ring(spec.ring, spec.model, spec.seq_k, spec.seq_v, f"step {step}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("G,d", [(4, 64), (8, 128), (16, 256), (32, 128)])
def test_windowed_attention_after_rollbacks(dt, G, d):
    """A speculative loop: k drafts appended (each attended), some rejected and rolled back, a
    correction appended. The windowed output at every draft step equals the oracle over the
    logical sequence as it stands (sinks + last W positions), with slack slots skipped."""
    B, Hkv, S, Wn, slack, k = 2, 2, 4, 48, 4, 4
    Hq = G * Hkv
    say(f"windowed after rollbacks {dt} G={G} d={d}")
    spec = _Spec(B, Hkv, d, S, Wn, slack, dt, seed=77)
    rng = np.random.default_rng(G * 100 + d)
    scale = 1.0 / math.sqrt(d)
    ws = W.workspace(B, Hq, Hkv, d, 1, spec.ring.capacity)
    spec.append(150)
    for it in range(6):
        for i in range(k):
            spec.append(1)
            q = synth.queries(91, it * k + i, B, 1, Hq, d, tdtype(dt), DEV)
            out = torch.full((B, 1, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
            lse = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device=DEV)
            W.wmtp_draft_attn_windowed(spec.ring, q, Hq, scale, out, lse, ws)
            ro, rl = oracle.draft_windowed(synth.host_array(q), ocode(dt), spec.logical_kv(),
                                           spec.model.n.tolist(), S, Wn, scale)
            compare(out, lse, ro, rl, dt, f"iteration {it} draft {i}")
        spec.rollback(rng.integers(0, k + 1, size=B).tolist())
        spec.append(1)  # the target's correction / bonus token
    _check_ring(spec.ring, spec.model, spec.seq_k, spec.seq_v, "end of loop")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("S,Wn,slack", [(4, 7, 3), (0, 7, 3), (2, 16, 9)])
def test_rollback_deeper_than_the_last_append(dt, S, Wn, slack):
    """Rollbacks that ask for more than was appended since the previous one (the device must stop
    where a later append overwrote a window slot): after each, the tags and bytes equal the host
    model's and the windowed read equals the oracle over the logical sequence."""
    B, Hkv, d, G = 3, 2, 128, 8
    Hq = G * Hkv
    say(f"deep rollbacks {dt} S={S} W={Wn} slack={slack}")
    spec = _Spec(B, Hkv, d, S, Wn, slack, dt, seed=53)
    rng = np.random.default_rng(S * 100 + Wn + slack)
    scale = 1.0 / math.sqrt(d)
    ws = W.workspace(B, Hq, Hkv, d, 1, spec.ring.capacity)
    spec.append(19)
    for step in range(16):
        spec.append(int(rng.integers(1, 3)))
        spec.rollback([slack, int(rng.integers(0, slack + 3)), slack + 1])
        _check_ring(spec.ring, spec.model, spec.seq_k, spec.seq_v, f"step {step}")
        q = synth.queries(97, step, B, 1, Hq, d, tdtype(dt), DEV)
        out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=DEV)
        lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)
        W.wmtp_draft_attn_windowed(spec.ring, q, Hq, scale, out, lse, ws)
        ro, rl = oracle.draft_windowed(synth.host_array(q), ocode(dt), spec.logical_kv(),
                                       spec.model.n.tolist(), S, Wn, scale)
        compare(out, lse, ro, rl, dt, f"step {step}")


def _logits(B, k, V, dt, seed, ties=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, k + 1, V), generator=g, dtype=torch.float32)
    if ties:  # copy each row's maximum to a second, later or earlier, index
        for b in range(B):
            for i in range(k + 1):
                j = int(torch.argmax(x[b, i]))
                x[b, i, (j + 1 + (b * 7 + i) % (V - 1)) % V] = x[b, i, j]
    return x.to(torch.bfloat16 if dt == "bf16" else torch.float32)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,k,V", [(1, 5, 151936), (3, 4, 4096), (4, 1, 4097), (2, 0, 50),
                                   (8, 7, 32000)])
def test_greedy_accept_exact(dt, B, k, V):
    say(f"greedy accept {dt} B={B} k={k} V={V}")
    x = _logits(B, k, V, dt, seed=B * 100 + k * 10 + V % 97)
    host = x.float().double().numpy()  # exact for bf16 and f32
    choice_ref = np.argmax(host, axis=2)
    rng = np.random.default_rng(V + k)
    draft = np.empty((B, k), dtype=np.int64)
    for b in range(B):  # accept a random prefix, then a mismatch (or all)
        a = int(rng.integers(0, k + 1))
        for i in range(k):
            draft[b, i] = choice_ref[b, i] if i < a else (choice_ref[b, i] + 1) % V
    ch_ref, acc_ref, nxt_ref, drop_ref = oracle.greedy_accept(host, draft)
    xd = x.to(DEV)
    dd = torch.tensor(draft, dtype=torch.int32, device=DEV)
    choice = torch.full((B, k + 1), -7, dtype=torch.int32, device=DEV)
    n_acc, nxt, drop = (torch.full((B,), -7, dtype=torch.int32, device=DEV) for _ in range(3))
    ws = W.accept_workspace(B, k, V)
    W.wmtp_greedy_accept(xd, k, dd, choice, n_acc, nxt, drop, ws)
    assert np.array_equal(choice.cpu().numpy(), ch_ref)
    assert np.array_equal(n_acc.cpu().numpy(), acc_ref)
    assert np.array_equal(nxt.cpu().numpy(), nxt_ref)
    assert np.array_equal(drop.cpu().numpy(), drop_ref)


def test_accept_feeds_rollback_on_device():
    """Verification outcome to ring state without the host: n_drop from wmtp_greedy_accept goes
    straight into wmtp_ring_rollback on the same stream."""
    B, Hkv, d, S, Wn, k, V = 4, 2, 128, 4, 32, 5, 1000
    say("accept -> rollback chain")
    spec = _Spec(B, Hkv, d, S, Wn, k, "bf16", seed=5)
    spec.append(100)
    spec.append(k)  # the k drafts
    x = _logits(B, k, V, "bf16", seed=9, ties=False)
    host = x.float().double().numpy()
    choice_ref = np.argmax(host, axis=2)
    draft = np.array([[choice_ref[b, i] if i < b else (choice_ref[b, i] + 3) % V for i in range(k)]
                      for b in range(B)])
    _, acc_ref, _, drop_ref = oracle.greedy_accept(host, draft)
    assert acc_ref.tolist() == [0, 1, 2, 3]
    choice = torch.empty((B, k + 1), dtype=torch.int32, device=DEV)
    n_acc, nxt, drop = (torch.empty((B,), dtype=torch.int32, device=DEV) for _ in range(3))
    W.wmtp_greedy_accept(x.to(DEV), k, torch.tensor(draft, dtype=torch.int32, device=DEV), choice,
                         n_acc, nxt, drop, W.accept_workspace(B, k, V))
    W.wmtp_ring_rollback(spec.ring, drop)
    for b in range(B):
        spec.model.rollback(b, int(drop_ref[b]))
        n = int(spec.model.n[b])
        spec.seq_k[b], spec.seq_v[b] = spec.seq_k[b][:, :n], spec.seq_v[b][:, :n]
    _check_ring(spec.ring, spec.model, spec.seq_k, spec.seq_v, "after accept + rollback")


# ------------------------------------------------------------------------------------------
# fused draft steps: append + attend in one call == the two calls, bit for bit
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["windowed", "windowed-slack", "full"])
@pytest.mark.parametrize("dt,d,G", [("bf16", 256, 16), ("bf16", 128, 8), ("f32", 64, 4),
                                    ("bf16", 128, 32)])  # G = 32: several row blocks
def test_fused_draft_step_equals_append_then_attend(form, dt, d, G):
    B, Hkv, S, Wn, steps = 2, 2, 4, 40, 6
    Hq = G * Hkv
    say(f"fused draft step {form} {dt} d={d} G={G}")
    lens = [130, 37]
    cap = max(lens) + steps + 8
    K, V = logical_kv(97, B, Hkv, d, max(lens) + steps, tdtype(dt))

    def make():
        if form == "full":
            c = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt), with_pos=True)
        else:
            c = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=3 if form == "windowed-slack" else 0)
        append_each(c, K, V, [0] * B, lens)
        return c

    fused, split = make(), make()
    scale = 1.0 / math.sqrt(d)
    ws1 = W.workspace(B, Hq, Hkv, d, 1, cap)
    ws2 = W.workspace(B, Hq, Hkv, d, 1, cap)
    for i in range(steps):
        kn = torch.stack([K[b, :, lens[b] + i:lens[b] + i + 1].permute(1, 0, 2) for b in range(B)]).contiguous()
        vn = torch.stack([V[b, :, lens[b] + i:lens[b] + i + 1].permute(1, 0, 2) for b in range(B)]).contiguous()
        q = synth.queries(98, i, B, 1, Hq, d, tdtype(dt), DEV)
        o1 = torch.full((B, 1, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        l1 = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device=DEV)
        o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
        W.wmtp_ring_append(split, kn, vn, 1)
        if form == "full":
            W.wmtp_draft_step_full(fused, kn, vn, q, Hq, scale, cap, o1, l1, ws1)
            W.wmtp_draft_attn_full(split, q, Hq, scale, cap, o2, l2, ws2)
        else:
            W.wmtp_draft_step_windowed(fused, kn, vn, q, Hq, scale, o1, l1, ws1)
            W.wmtp_draft_attn_windowed(split, q, Hq, scale, o2, l2, ws2)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {i}: outputs differ"
        for name in ("k", "v", "pos", "seq_len"):
            assert torch.equal(getattr(fused, name), getattr(split, name)), f"step {i}: {name}"
        n = [lens[b] + i + 1 for b in range(B)]
        kv = oracle_kv_for(K, V, dt)
        if form == "full":
            ro, rl = oracle.draft_full(synth.host_array(q), ocode(dt), kv, n, scale)
        else:
            ro, rl = oracle.draft_windowed(synth.host_array(q), ocode(dt), kv, n, S, Wn, scale)
        compare(o1, l1, ro, rl, dt, f"fused step {i}")


def oracle_kv_for(K, V, dt):
    return oracle.contiguous_kv(synth.host_array(K), synth.host_array(V), ocode(dt))


@pytest.mark.parametrize("dt,d,Hq,Hkv,m", [
    ("bf16", 128, 32, 2, 4),    # 64 rows: cooperative kernel, fused
    ("bf16", 128, 32, 2, 6),    # 96 rows: two row blocks per wavefront
    ("bf16", 64, 32, 2, 5),
    ("bf16", 256, 32, 2, 3),    # 48 rows at head_dim 256
    ("bf16", 128, 64, 2, 3),    # 96 rows
    ("bf16", 128, 32, 1, 8),    # 256 rows: two row chunks, both read the new rows
    ("f32", 64, 8, 2, 6),       # 24 rows, fp32: key-split kernel (two row blocks), append first
    ("f32", 64, 16, 2, 8),      # 64 rows, fp32: cooperative kernel, fused
    ("bf16", 128, 8, 2, 2),     # 8 rows: split kernel, append first
])
def test_fused_verify_step_equals_append_then_verify(dt, d, Hq, Hkv, m):
    B = 2
    say(f"fused verify step {dt} d={d} Hq={Hq} Hkv={Hkv} m={m}")
    lens = [3000, 517]
    steps = 3
    cap = max(lens) + steps * m + 24
    K, V = logical_kv(107, B, Hkv, d, max(lens) + steps * m, tdtype(dt))

    def make():
        c = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt), with_pos=True)
        append_each(c, K, V, [0] * B, lens)
        return c

    fused, split = make(), make()
    scale = 1.0 / math.sqrt(d)
    ws1 = W.workspace(B, Hq, Hkv, d, m, cap)
    ws2 = W.workspace(B, Hq, Hkv, d, m, cap)
    for i in range(steps):
        cur = [lens[b] + i * m for b in range(B)]
        kn = torch.stack([K[b, :, cur[b]:cur[b] + m].permute(1, 0, 2) for b in range(B)]).contiguous()
        vn = torch.stack([V[b, :, cur[b]:cur[b] + m].permute(1, 0, 2) for b in range(B)]).contiguous()
        q = synth.queries(108, i, B, m, Hq, d, tdtype(dt), DEV)
        o1 = torch.full((B, m, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        l1 = torch.full((B, m, Hq), float("nan"), dtype=torch.float32, device=DEV)
        o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
        W.wmtp_verify_step(fused, kn, vn, q, m, Hq, scale, cap, o1, l1, ws1)
        W.wmtp_ring_append(split, kn, vn, m)
        W.wmtp_verify_attn(split, q, m, Hq, scale, cap, o2, l2, ws2)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {i}: outputs differ"
        for name in ("k", "v", "pos", "seq_len"):
            assert torch.equal(getattr(fused, name), getattr(split, name)), f"step {i}: {name}"
        n = [c + m for c in cur]
        ro, rl = oracle.verify(synth.host_array(q), ocode(dt), oracle_kv_for(K, V, dt), n, scale)
        compare(o1, l1, ro, rl, dt, f"fused verify step {i}")
