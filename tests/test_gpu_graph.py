"""A decode iteration captured in a HIP graph and replayed must give, replay after replay, the
same bytes as the same calls launched one by one: ring and cache contents, outputs and
log-sum-exps. The library launches kernels only (no memset or copy nodes), reads every length
from device memory, and keeps no host-side state between calls, which is what makes its calls
capturable; replays are interleaved with unrelated eager work and synchronisations."""
import math

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
