"""A decode iteration captured in a HIP graph and replayed must give, replay after replay, the
same bytes as the same calls launched one by one: ring and cache contents, outputs and
log-sum-exps. The library launches kernels only (no memset or copy nodes), reads every length
from device memory, and keeps no host-side state between calls, which is what makes its calls
capturable; replays are interleaved with unrelated eager work and synchronisations."""
import math

import numpy as np
import pytest
import torch

from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import DEV, append_all, logical_kv, say

pytestmark = pytest.mark.gpu


class _Iteration:
    """Caches and buffers of one decode iteration: k draft steps (ring append + windowed
    attention, contiguous append + full attention) and one verification of m candidates."""

    def __init__(self, K, V, Kt, Vt, L, S, Wn, Hq, m, k, cap):
        B, Hkv, _, d = K.shape
        dt = K.dtype
        self.k, self.m, self.Hq, self.cap = k, m, Hq, cap
        self.ring = W.KVCache.ring(B, Hkv, d, S, Wn, dt)
        self.full = W.KVCache.contiguous(B, Hkv, d, cap, dt)
        self.tgt = W.KVCache.contiguous(B, Hkv, d, cap, dt)
        for c, kk, vv in ((self.ring, K, V), (self.full, K, V), (self.tgt, Kt, Vt)):
            append_all(c, kk, vv, [0] * B, L)
        self.scale = 1.0 / math.sqrt(d)
        self.out_w = torch.zeros((k, B, 1, Hq, d), dtype=torch.float32, device=DEV)
        self.lse_w = torch.zeros((k, B, 1, Hq), dtype=torch.float32, device=DEV)
        self.out_f = torch.zeros_like(self.out_w)
        self.lse_f = torch.zeros_like(self.lse_w)
        self.out_v = torch.zeros((B, m, Hq, d), dtype=torch.float32, device=DEV)
        self.lse_v = torch.zeros((B, m, Hq), dtype=torch.float32, device=DEV)
        self.ws_w = W.workspace(B, Hq, Hkv, d, 1, S + Wn)
        self.ws_f = W.workspace(B, Hq, Hkv, d, 1, cap)
        self.ws_v = W.workspace(B, Hq, Hkv, d, m, cap)

    def run(self, draft_k, draft_v, draft_q, cand_k, cand_v, ver_q):
        for i in range(self.k):
            kn, vn = draft_k[i], draft_v[i]
            W.wmtp_ring_append(self.ring, kn, vn, 1)
            W.wmtp_draft_attn_windowed(self.ring, draft_q[i], self.Hq, self.scale,
                                       self.out_w[i], self.lse_w[i], self.ws_w)
            W.wmtp_ring_append(self.full, kn, vn, 1)
            W.wmtp_draft_attn_full(self.full, draft_q[i], self.Hq, self.scale, self.cap,
                                   self.out_f[i], self.lse_f[i], self.ws_f)
        W.wmtp_ring_append(self.tgt, cand_k, cand_v, self.m)
        W.wmtp_verify_attn(self.tgt, ver_q, self.m, self.Hq, self.scale, self.cap,
                           self.out_v, self.lse_v, self.ws_v)

    def state(self):
        cut = lambda c: [c.k.clone(), c.v.clone(), c.seq_len.clone()] + \
            ([] if c.pos is None else [c.pos.clone()])
        return (cut(self.ring) + cut(self.full) + cut(self.tgt) +
                [t.clone() for t in (self.out_w, self.lse_w, self.out_f, self.lse_f,
                                     self.out_v, self.lse_v)])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_graph_replay_matches_eager(dt):
    B, Hq, Hkv, d, S, Wn, m, k = 2, 16, 2, 128, 4, 64, 4, 3
    L, replays = 3000, 3
    cap = L + (replays + 1) * max(k, m) + 16
    say(f"graph replay vs eager {dt} B={B} Hq={Hq} Hkv={Hkv} d={d} S={S} W={Wn} L={L} k={k} m={m}")
    K, V = logical_kv(2101, B, Hkv, d, L + k, dt)
    Kt, Vt = logical_kv(2102, B, Hkv, d, L + m, dt)
    # per draft step, the token of every sequence: [B][1][Hkv][d]
    draft_k = [torch.stack([K[b, :, L + i:L + i + 1].permute(1, 0, 2) for b in range(B)]).contiguous()
               for i in range(k)]
    draft_v = [torch.stack([V[b, :, L + i:L + i + 1].permute(1, 0, 2) for b in range(B)]).contiguous()
               for i in range(k)]
    cand_k = torch.stack([Kt[b, :, L:L + m].permute(1, 0, 2) for b in range(B)]).contiguous()
    cand_v = torch.stack([Vt[b, :, L:L + m].permute(1, 0, 2) for b in range(B)]).contiguous()
    draft_q = [synth.queries(2103, i, B, 1, Hq, d, dt, DEV) for i in range(k)]
    ver_q = synth.queries(2104, 0, B, m, Hq, d, dt, DEV)
    inputs = (draft_k, draft_v, draft_q, cand_k, cand_v, ver_q)

    eager = _Iteration(K, V, Kt, Vt, L, S, Wn, Hq, m, k, cap)
    graphed = _Iteration(K, V, Kt, Vt, L, S, Wn, Hq, m, k, cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run(*inputs)
    torch.cuda.synchronize()
    # capture launches nothing: the graphed caches still hold the prefill only
    assert torch.equal(graphed.full.seq_len, eager.full.seq_len)

    side = _Iteration(K, V, Kt, Vt, L, S, Wn, Hq, m, k, cap)
    for r in range(replays):
        say(f"  replay {r}")
        eager.run(*inputs)
        g.replay()
        # unrelated eager library work and torch ops between replays
        side.run(*inputs)
        junk = torch.randn(1 << 16, device=DEV).cumsum(0)
        torch.cuda.synchronize()
        del junk
        want, got = eager.state(), graphed.state()
        for i, (a, b) in enumerate(zip(want, got)):
            assert torch.equal(a, b), f"replay {r}: tensor {i} differs from the eager run"
        n = int(graphed.full.seq_len[0].item())
        assert n == L + (r + 1) * k, f"replay {r}: contiguous length {n}"


def test_graph_replay_of_a_speculative_iteration():
    """The whole speculative iteration as a serving engine would capture it: k fused draft steps
    (windowed on a ring with slack, full on a contiguous cache), the target's append and
    verification, greedy acceptance on device logits and the rollbacks driven by its device-side
    n_drop. Replays equal the eager calls bit for bit, replay after replay."""
    dt = torch.bfloat16
    B, Hq, Hkv, d, S, Wn, k, V = 2, 16, 2, 128, 4, 64, 3, 512
    L, replays = 2000, 3
    cap = L + (replays + 2) * (k + 1) + 16
    say(f"graph replay of a speculative iteration B={B} d={d} k={k}")
    K, Vv = logical_kv(2201, B, Hkv, d, L, dt)
    Kt, Vt = logical_kv(2202, B, Hkv, d, L, dt)
    tok_k = [torch.stack([synth.token_rows(2203, synth.KNEW_ID, b, i, i + 1, Hkv, d, dt, DEV)
                          for b in range(B)]) for i in range(k)]
    tok_v = [torch.stack([synth.token_rows(2203, synth.VNEW_ID, b, i, i + 1, Hkv, d, dt, DEV)
                          for b in range(B)]) for i in range(k)]
    cand_k = torch.stack([synth.token_rows(2204, synth.KNEW_ID, b, 0, k + 1, Hkv, d, dt, DEV)
                          for b in range(B)])
    cand_v = torch.stack([synth.token_rows(2204, synth.VNEW_ID, b, 0, k + 1, Hkv, d, dt, DEV)
                          for b in range(B)])
    q3 = [synth.queries(2205, i, B, 1, Hq, d, dt, DEV) for i in range(k)]
    q4 = synth.queries(2206, 0, B, k + 1, Hq, d, dt, DEV)
    g0 = torch.Generator().manual_seed(7)
    logits = torch.randn((B, k + 1, V), generator=g0).to(dt).to(DEV)
    choice = np.argmax(logits.float().cpu().numpy(), axis=2)  # first maximum, as the rule says
    # sequence 0 keeps its first draft, sequence 1 keeps none
    drafts = torch.tensor([[choice[0, 0], (choice[0, 1] + 1) % V, choice[0, 2]],
                           [(choice[1, i] + 1) % V for i in range(k)]],
                          dtype=torch.int32, device=DEV)

    class It:
        def __init__(self):
            self.ring = W.KVCache.ring(B, Hkv, d, S, Wn, dt, slack=k)
            self.full = W.KVCache.contiguous(B, Hkv, d, cap, dt, with_pos=True)
            self.tgt = W.KVCache.contiguous(B, Hkv, d, cap, dt)
            append_all(self.ring, K, Vv, [0] * B, L)
            append_all(self.full, K, Vv, [0] * B, L)
            append_all(self.tgt, Kt, Vt, [0] * B, L)
            self.ow = torch.zeros((k, B, 1, Hq, d), dtype=torch.float32, device=DEV)
            self.lw = torch.zeros((k, B, 1, Hq), dtype=torch.float32, device=DEV)
            self.of, self.lf = torch.zeros_like(self.ow), torch.zeros_like(self.lw)
            self.ov = torch.zeros((B, k + 1, Hq, d), dtype=torch.float32, device=DEV)
            self.lv = torch.zeros((B, k + 1, Hq), dtype=torch.float32, device=DEV)
            self.choice = torch.zeros((B, k + 1), dtype=torch.int32, device=DEV)
            self.acc, self.nxt, self.drop = (torch.zeros((B,), dtype=torch.int32, device=DEV)
                                             for _ in range(3))
            self.ws_w = W.workspace(B, Hq, Hkv, d, 1, self.ring.capacity)
            self.ws_f = W.workspace(B, Hq, Hkv, d, 1, cap)
            self.ws_v = W.workspace(B, Hq, Hkv, d, k + 1, cap)
            self.ws_a = W.accept_workspace(B, k, V)

        def run(self):
            for i in range(k):
                W.wmtp_draft_step_windowed(self.ring, tok_k[i], tok_v[i], q3[i], Hq, 0.09,
                                           self.ow[i], self.lw[i], self.ws_w)
                W.wmtp_draft_step_full(self.full, tok_k[i], tok_v[i], q3[i], Hq, 0.09, cap,
                                       self.of[i], self.lf[i], self.ws_f)
            W.wmtp_ring_append(self.tgt, cand_k, cand_v, k + 1)
            W.wmtp_verify_attn(self.tgt, q4, k + 1, Hq, 0.09, cap, self.ov, self.lv, self.ws_v)
            W.wmtp_greedy_accept(logits, k, drafts, self.choice, self.acc, self.nxt, self.drop,
                                 self.ws_a)
            W.wmtp_ring_rollback(self.ring, self.drop)
            W.wmtp_ring_rollback(self.full, self.drop)
            W.wmtp_ring_rollback(self.tgt, self.drop)

        def state(self):
            out = []
            for c in (self.ring, self.full, self.tgt):
                out += [c.k.clone(), c.v.clone(), c.seq_len.clone()]
                if c.pos is not None:
                    out.append(c.pos.clone())
            return out + [t.clone() for t in (self.ow, self.lw, self.of, self.lf, self.ov, self.lv,
                                              self.choice, self.acc, self.nxt, self.drop)]

    eager, graphed = It(), It()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    side = It()
    for r in range(replays):
        say(f"  replay {r}")
        eager.run()
        g.replay()
        side.run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager.state(), graphed.state())):
            assert torch.equal(a, b), f"replay {r}: tensor {i} differs from the eager run"
        assert graphed.acc.tolist() == [1, 0]
        assert graphed.ring.seq_len.tolist() == [L + r + 1, L]
        assert graphed.tgt.seq_len.tolist() == [L + 2 * (r + 1), L + r + 1]


def test_graph_replay_of_fused_verification_and_masw():
    """The fused verification step on the cooperative kernel (its candidates stored by one
    workgroup, the length advanced by the merge) and the MASW-style step (two reads, one merge),
    captured together: replays equal the eager calls bit for bit, replay after replay."""
    dt = torch.bfloat16
    B, Hq, Hkv, d, m, S, Wn, n_slots = 2, 32, 2, 128, 4, 4, 64, 40
    L, replays = 1500, 3
    cap = L + (replays + 2) * m + 16
    say(f"graph replay of the fused verification and the MASW step B={B} Hq={Hq} m={m}")
    K, Vv = logical_kv(2301, B, Hkv, d, L, dt)
    SK, SV = logical_kv(2302, B, Hkv, d, n_slots, dt)
    cand_k = torch.stack([synth.token_rows(2303, synth.KNEW_ID, b, 0, m, Hkv, d, dt, DEV)
                          for b in range(B)])
    cand_v = torch.stack([synth.token_rows(2303, synth.VNEW_ID, b, 0, m, Hkv, d, dt, DEV)
                          for b in range(B)])
    qv = synth.queries(2304, 0, B, m, Hq, d, dt, DEV)
    qd = synth.queries(2305, 0, B, 1, Hq // 2, d, dt, DEV)

    class It:
        def __init__(self):
            self.tgt = W.KVCache.contiguous(B, Hkv, d, cap, dt)
            append_all(self.tgt, K, Vv, [0] * B, L)
            self.ring = W.KVCache.ring(B, Hkv, d, S, Wn, dt)
            append_all(self.ring, K, Vv, [0] * B, L)
            self.slots = W.KVCache.contiguous(B, Hkv, d, n_slots + 8, dt)
            append_all(self.slots, SK, SV, [0] * B, n_slots)
            self.ov = torch.zeros((B, m, Hq, d), dtype=torch.float32, device=DEV)
            self.lv = torch.zeros((B, m, Hq), dtype=torch.float32, device=DEV)
            self.om = torch.zeros((B, 1, Hq // 2, d), dtype=torch.float32, device=DEV)
            self.lm = torch.zeros((B, 1, Hq // 2), dtype=torch.float32, device=DEV)
            self.ws_v = W.workspace(B, Hq, Hkv, d, m, cap)
            self.ws_m = W.masw_workspace(B, Hq // 2, Hkv, d, self.ring.capacity, n_slots + 8)

        def run(self):
            W.wmtp_verify_step(self.tgt, cand_k, cand_v, qv, m, Hq, 0.09, cap, self.ov, self.lv,
                               self.ws_v)
            W.wmtp_draft_attn_masw(self.ring, self.slots, qd, Hq // 2, 0.09, n_slots + 8, self.om,
                                   self.lm, self.ws_m)

        def state(self):
            out = []
            for c in (self.tgt, self.ring, self.slots):
                out += [c.k.clone(), c.v.clone(), c.seq_len.clone()]
            return out + [t.clone() for t in (self.ov, self.lv, self.om, self.lm)]

    eager, graphed = It(), It()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    side = It()
    for r in range(replays):
        say(f"  replay {r}")
        eager.run()
        g.replay()
        side.run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager.state(), graphed.state())):
            assert torch.equal(a, b), f"replay {r}: tensor {i} differs from the eager run"
        assert graphed.tgt.seq_len.tolist() == [L + (r + 1) * m] * B
