"""GPU parity of the HIP path (through the C ABI) against the float64 oracle, at sizes the oracle
finishes in seconds: several 16-key tiles, several splits, ragged tails, and the edge cases of
the sink/window/causal sets. Ring contents and position tags must match bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth
from gpu_common import (DEV, TOL, append_all, append_each, compare, logical_kv, ocode,
                        oracle_kv, run_full, run_verify, run_windowed, say, select, tdtype)

pytestmark = pytest.mark.gpu


def _check_ring(ring: W.KVCache, model: oracle.RingModel, kv: oracle.LogicalKV, what: str):
    tags = ring.pos.cpu().numpy().astype(np.int64)
    assert np.array_equal(tags, model.tags), f"{what}: position tags differ"
    assert np.array_equal(ring.seq_len.cpu().numpy().astype(np.int64), model.n), f"{what}: seq_len"
    rk, rv = oracle.ring_expected(model, kv)
    hk, hv = synth.host_array(ring.k), synth.host_array(ring.v)
    for b in range(ring.batch):
        occ = model.occupied_slots(b)
        assert np.array_equal(hk[b][:, occ], rk[b][:, occ]), f"{what}: K bytes of sequence {b}"
        assert np.array_equal(hv[b][:, occ], rv[b][:, occ]), f"{what}: V bytes of sequence {b}"


# ------------------------------------------------------------------------------------------
# ring append: bit-exact against the host ring model
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("S,Wn", [(4, 16), (0, 7), (3, 1), (4, 256)])
def test_ring_append_bitexact(dt, d, S, Wn):
    B, Hkv = 3, 2
    say(f"ring append {dt} d={d} S={S} W={Wn}")
    total = 3 * (S + Wn) + 700
    K, V = logical_kv(11, B, Hkv, d, total, tdtype(dt))
    kv = oracle_kv(K, V, dt)
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt))
    model = oracle.RingModel(B, S, Wn)
    lens = [0] * B
    # ragged prefixes (one call per sequence), then common appends of assorted sizes
    first = [1, S + Wn + 5, 2 * (S + Wn) + 3]
    append_each(ring, K, V, lens, first)
    for b, t in enumerate(first):
        model.append(b, t)
        lens[b] += t
    _check_ring(ring, model, kv, "after ragged prefill")
    for t in [1, 1, 3, Wn + 2, 1, S + 1, 2 * Wn + 7, 1]:
        if max(lens) + t > total:
            break
        append_all(ring, K, V, lens, t)
        for b in range(B):
            model.append(b, t)
            lens[b] += t
        _check_ring(ring, model, kv, f"after append of {t}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_contiguous_append_and_overflow(dt):
    B, Hkv, d, cap = 2, 2, 128, 300
    say(f"contiguous append {dt}")
    K, V = logical_kv(12, B, Hkv, d, cap + 40, tdtype(dt))
    cache = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt), with_pos=True)
    append_each(cache, K, V, [0, 0], [250, 17])
    append_all(cache, K, V, [250, 17], 30)  # sequence 0 reaches 280 of 300
    append_all(cache, K, V, [280, 47], 30)  # sequence 0 would reach 310: positions >= 300 dropped
    torch.cuda.synchronize()
    n = cache.seq_len.cpu().tolist()
    assert n == [310, 77]
    hk = synth.host_array(cache.k)
    exp = synth.host_array(K)
    assert np.array_equal(hk[0][:, :cap], exp[0][:, :cap])  # positions >= capacity dropped
    assert np.array_equal(hk[1][:, :77], exp[1][:, :77])
    pos = cache.pos.cpu().numpy()
    assert np.array_equal(pos[0], np.arange(cap))
    assert np.array_equal(pos[1][:77], np.arange(77)) and np.all(pos[1][77:] == -1)
    # the API refuses a single append larger than a contiguous cache
    kn = torch.zeros((B, cap + 1, Hkv, d), dtype=tdtype(dt), device=DEV)
    assert W.wmtp_ring_append(cache, kn, kn, cap + 1, check=False) == W.WMTP_ERR_CAPACITY


# ------------------------------------------------------------------------------------------
# windowed draft attention over the ring vs the oracle over the logical sequence
# ------------------------------------------------------------------------------------------
WIN_CASES = [
    # dt, d, Hq, Hkv, S, W, lens (ragged batch)
    ("f32", 64, 8, 2, 4, 256, [1, 3, 4, 5]),
    ("f32", 64, 8, 2, 4, 256, [259, 260, 261, 1000]),
    ("f32", 128, 4, 4, 0, 33, [1, 32, 33, 34, 500]),
    ("f32", 256, 16, 2, 2, 64, [65, 66, 67, 900]),
    ("bf16", 64, 4, 1, 4, 100, [3, 104, 105, 333]),
    ("bf16", 128, 32, 4, 4, 2048, [2051, 2052, 2053, 6000]),
    ("bf16", 128, 16, 2, 1, 1, [1, 2, 3, 50]),
    ("bf16", 256, 32, 2, 4, 512, [100, 516, 517, 3000]),
    ("bf16", 128, 48, 3, 4, 64, [70, 68]),
]


@pytest.mark.parametrize("dt,d,Hq,Hkv,S,Wn,lens", WIN_CASES)
def test_windowed_parity(dt, d, Hq, Hkv, S, Wn, lens):
    B = len(lens)
    say(f"windowed {dt} d={d} Hq={Hq} Hkv={Hkv} S={S} W={Wn} lens={lens}")
    K, V = logical_kv(21, B, Hkv, d, max(lens), tdtype(dt))
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt))
    # prefill all but the last token per sequence, then append one draft token to all
    pre = [n - 1 for n in lens]
    append_each(ring, K, V, [0] * B, pre)
    append_all(ring, K, V, pre, 1)
    q = synth.queries(22, 0, B, 1, Hq, d, tdtype(dt), DEV)
    scale = 1.0 / math.sqrt(d)
    out, lse = run_windowed(ring, q, Hq, scale)
    ref_o, ref_l = oracle.draft_windowed(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), lens,
                                         S, Wn, scale)
    compare(out, lse, ref_o, ref_l, dt, "windowed")


# ------------------------------------------------------------------------------------------
# full draft attention over a contiguous cache
# ------------------------------------------------------------------------------------------
FULL_CASES = [
    ("f32", 64, 8, 2, [1, 15, 16, 17, 4097]),
    ("f32", 128, 8, 8, [33, 1000]),
    ("f32", 256, 4, 1, [5000]),
    ("bf16", 64, 16, 2, [7, 999]),
    ("bf16", 128, 32, 4, [1, 2049, 7777]),
    ("bf16", 256, 32, 2, [12345, 300]),
    ("bf16", 128, 8, 8, [64, 65]),
]


@pytest.mark.parametrize("dt,d,Hq,Hkv,lens", FULL_CASES)
def test_full_parity(dt, d, Hq, Hkv, lens):
    B = len(lens)
    say(f"full {dt} d={d} Hq={Hq} Hkv={Hkv} lens={lens}")
    cap = max(lens) + 37
    K, V = logical_kv(31, B, Hkv, d, max(lens), tdtype(dt))
    cache = W.KVCache.contiguous(B, Hkv, d, cap, tdtype(dt))
    append_each(cache, K, V, [0] * B, lens)
    q = synth.queries(32, 0, B, 1, Hq, d, tdtype(dt), DEV)
    scale = 1.0 / math.sqrt(d)
    ref_o, ref_l = oracle.draft_full(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), lens,
                                     scale)
    # the host bound only sizes the launch: any bound >= every length gives the same result
    for bound in sorted({max(lens), cap}):
        out, lse = run_full(cache, q, Hq, scale, bound)
        compare(out, lse, ref_o, ref_l, dt, f"full (max_seq_len={bound})")


def test_full_bound_below_length_reads_nothing_beyond():
    """max_seq_len < seq_len: keys at or past the bound are never read (result = prefix)."""
    dt, d, Hq, Hkv, n, bound = "bf16", 128, 8, 2, 900, 700
    say("full with a short host bound")
    K, V = logical_kv(33, 1, Hkv, d, n, tdtype(dt))
    cache = W.KVCache.contiguous(1, Hkv, d, n, tdtype(dt))
    append_each(cache, K, V, [0], [n])
    q = synth.queries(34, 0, 1, 1, Hq, d, tdtype(dt), DEV)
    out, lse = run_full(cache, q, Hq, 0.1, bound)
    ref_o, ref_l = oracle.draft_full(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), [bound],
                                     0.1)
    compare(out, lse, ref_o, ref_l, dt, "full clamped to the bound")


# ------------------------------------------------------------------------------------------
# verification: m candidates, causal among themselves
# ------------------------------------------------------------------------------------------
# rows per KV head = m * Hq / Hkv; the key-split kernel takes up to 48 (32 for bf16 at head_dim
# 256 and fp32 at 128, 16 for fp32 at 256), the cooperative kernel the rest
VERIFY_CASES = [
    ("bf16", 128, 32, 2, 4, [5000, 64]),  # 64 rows: cooperative
    ("bf16", 128, 16, 2, 1, [300]),       # 8 rows: key-split
    ("bf16", 64, 8, 2, 6, [777, 6]),      # 24 rows: key-split, two row blocks
    ("bf16", 256, 16, 2, 2, [1500]),      # 16 rows: key-split
    ("bf16", 256, 32, 2, 3, [900]),       # 48 rows: cooperative (past 32 at head_dim 256)
    ("bf16", 256, 32, 2, 6, [901]),       # 96 rows: cooperative, two row chunks
    ("f32", 64, 8, 2, 4, [4097, 2]),      # 16 rows: key-split
    ("f32", 128, 8, 1, 3, [999]),         # 24 rows: key-split, two row blocks
    ("bf16", 128, 8, 4, 16, [2000]),      # 32 rows: key-split, two row blocks
    ("bf16", 128, 16, 2, 6, [1300, 33]),  # 48 rows: key-split, three row blocks
    ("f32", 64, 8, 2, 12, [700]),         # 48 rows: key-split, three row blocks, fp32
    ("f32", 128, 16, 2, 6, [650]),        # 48 rows: cooperative (past 32 for fp32 at 128)
    ("bf16", 128, 32, 2, 6, [3000, 77]),  # 96 rows: cooperative, two row blocks per wavefront
    ("bf16", 128, 16, 1, 8, [2500]),      # 128 rows: cooperative
    ("bf16", 64, 32, 2, 5, [1234]),       # 80 rows at head_dim 64: cooperative
]


@pytest.mark.parametrize("dt,d,Hq,Hkv,m,lens", VERIFY_CASES)
def test_verify_parity(dt, d, Hq, Hkv, m, lens):
    B = len(lens)
    say(f"verify {dt} d={d} Hq={Hq} Hkv={Hkv} m={m} lens={lens}")
    K, V = logical_kv(41, B, Hkv, d, max(lens), tdtype(dt))
    cache = W.KVCache.contiguous(B, Hkv, d, max(lens) + 8, tdtype(dt))
    append_each(cache, K, V, [0] * B, lens)
    q = synth.queries(42, 0, B, m, Hq, d, tdtype(dt), DEV)
    scale = 1.0 / math.sqrt(d)
    out, lse = run_verify(cache, q, Hq, scale, max(lens))
    ref_o, ref_l = oracle.verify(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), lens, scale)
    compare(out, lse, ref_o, ref_l, dt, "verify")


@pytest.mark.parametrize("m,Hq", [(1, 8), (4, 32)])
def test_loose_host_bound(m, Hq):
    """A host bound far above every length sizes the launch for 64K keys: most workgroups then
    have no tile of a short sequence (they request clamped rows and contribute nothing)."""
    dt, d, Hkv, lens, bound = "bf16", 128, 2, [300, 4100], 65536
    B = len(lens)
    say(f"loose host bound {bound}: m={m} Hq={Hq} lens={lens}")
    K, V = logical_kv(45, B, Hkv, d, max(lens), tdtype(dt))
    cache = W.KVCache.contiguous(B, Hkv, d, bound + 16, tdtype(dt))
    append_each(cache, K, V, [0] * B, lens)
    q = synth.queries(46, 0, B, m, Hq, d, tdtype(dt), DEV)
    if m == 1:
        out, lse = run_full(cache, q, Hq, 0.1, bound)
        ref_o, ref_l = oracle.draft_full(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), lens,
                                         0.1)
    else:
        out, lse = run_verify(cache, q, Hq, 0.1, bound)
        ref_o, ref_l = oracle.verify(synth.host_array(q), ocode(dt), oracle_kv(K, V, dt), lens, 0.1)
    compare(out, lse, ref_o, ref_l, dt, "loose host bound")


# ------------------------------------------------------------------------------------------
# properties that hold on the device
# ------------------------------------------------------------------------------------------
def test_windowed_equals_full_when_window_covers_all():
    dt, d, Hq, Hkv, S, Wn, n = "f32", 64, 8, 2, 4, 256, 257
    say("windowed == full at S+W >= n")
    K, V = logical_kv(51, 1, Hkv, d, n, tdtype(dt))
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, tdtype(dt))
    cache = W.KVCache.contiguous(1, Hkv, d, n, tdtype(dt))
    append_each(ring, K, V, [0], [n])
    append_each(cache, K, V, [0], [n])
    q = synth.queries(52, 0, 1, 1, Hq, d, tdtype(dt), DEV)
    ow, lw = run_windowed(ring, q, Hq, 0.125)
    of, lf = run_full(cache, q, Hq, 0.125, n)
    assert torch.max(torch.abs(ow - of)).item() <= TOL[dt]
    assert torch.max(torch.abs(lw - lf)).item() <= TOL[dt]


def test_deterministic():
    dt, d, Hq, Hkv, n = "bf16", 128, 32, 2, 20000
    say("determinism")
    K, V = logical_kv(61, 1, Hkv, d, n, tdtype(dt))
    cache = W.KVCache.contiguous(1, Hkv, d, n, tdtype(dt))
    append_each(cache, K, V, [0], [n])
    q = synth.queries(62, 0, 1, 4, Hq, d, tdtype(dt), DEV)
    a = run_verify(cache, q, Hq, 0.1, n)
    b = run_verify(cache, q, Hq, 0.1, n)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_sequences_give_zero_and_minus_inf():
    dt, d, Hq, Hkv = "bf16", 128, 8, 2
    say("empty sequences")
    ring = W.KVCache.ring(2, Hkv, d, 4, 16, tdtype(dt))
    q = synth.queries(71, 0, 2, 1, Hq, d, tdtype(dt), DEV)
    out, lse = run_windowed(ring, q, Hq, 0.1)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    cache = W.KVCache.contiguous(2, Hkv, d, 64, tdtype(dt))
    K, V = logical_kv(72, 2, Hkv, d, 2, tdtype(dt))
    append_each(cache, K, V, [0, 0], [0, 2])  # sequence 0 stays empty, sequence 1 holds 2 tokens
    qv = synth.queries(73, 0, 2, 4, Hq, d, tdtype(dt), DEV)
    out, lse = run_verify(cache, qv, Hq, 0.1, 64)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    # sequence 1: candidates 0 and 1 see nothing (positions -2, -1), 2 and 3 see 1 and 2 tokens
    assert torch.all(out[1, :2] == 0) and torch.all(torch.isneginf(lse[1, :2]))
    ref_o, ref_l = oracle.verify(synth.host_array(qv[1:]), ocode(dt), oracle_kv(K[1:], V[1:], dt),
                                 [2], 0.1)
    compare(out[1:], lse[1:], ref_o, ref_l, dt, "verify with n < m")


def test_null_lse_gives_the_same_outputs():
    """lse is optional: with a NULL lse every read writes the same outputs, bit for bit."""
    dt, d, Hkv, B = "bf16", 128, 2, 2
    say("null lse: windowed, full and verify (split and cooperative kernels)")
    K, V = logical_kv(47, B, Hkv, d, 3000, tdtype(dt))
    ring = W.KVCache.ring(B, Hkv, d, 4, 256, tdtype(dt))
    append_each(ring, K, V, [0] * B, [3000, 700])
    cache = W.KVCache.contiguous(B, Hkv, d, 3008, tdtype(dt))
    append_each(cache, K, V, [0] * B, [3000, 700])
    # 8 and 32 rows (key-split: one and two row blocks) and 64 rows (cooperative) per KV head
    for Hq, m in ((16, 1), (16, 4), (16, 8)):
        q = synth.queries(48, 0, B, m, Hq, d, tdtype(dt), DEV)
        calls = [("verify", lambda o, l: W.wmtp_verify_attn(
            cache, q, m, Hq, 0.1, 3000, o, l, W.workspace(B, Hq, Hkv, d, m, 3000)))]
        if m == 1:
            calls += [
                ("windowed", lambda o, l: W.wmtp_draft_attn_windowed(
                    ring, q, Hq, 0.1, o, l, W.workspace(B, Hq, Hkv, d, 1, ring.capacity))),
                ("full", lambda o, l: W.wmtp_draft_attn_full(
                    cache, q, Hq, 0.1, 3000, o, l, W.workspace(B, Hq, Hkv, d, 1, 3000)))]
        for name, call in calls:
            o1 = torch.full((B, m, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
            l1 = torch.empty((B, m, Hq), dtype=torch.float32, device=DEV)
            o2 = torch.full_like(o1, float("nan"))
            call(o1, l1)
            call(o2, None)
            assert torch.equal(o1, o2), f"{name} (m={m}): outputs differ without lse"


# ------------------------------------------------------------------------------------------
# rows past a sequence's length are never attended: whatever bytes they hold (NaN here), the
# results do not change. Short sequences under a larger host bound make the first tiles straddle
# the end (key-split kernel) and the staged tiles run past it (cooperative kernel).
# ------------------------------------------------------------------------------------------
def _poison(cache: W.KVCache, lens, from_offset: int = 0):
    """Copy of `cache` whose rows (ring: slots) at or past each length hold NaN bytes."""
    c = W.KVCache(cache.k.clone(), cache.v.clone(),
                  None if cache.pos is None else cache.pos.clone(), cache.seq_len.clone(),
                  cache.batch, cache.n_kv_heads, cache.head_dim, cache.capacity, cache.sink,
                  cache.window, cache.dtype)
    for b, n in enumerate(lens):
        r0 = n + from_offset
        if r0 < cache.capacity:
            c.k[b, :, r0:] = float("nan")
            c.v[b, :, r0:] = float("nan")
    return c


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 256), ("f32", 64), ("f32", 128)])
def test_bytes_past_the_length_do_not_reach_results(dt, d):
    Hkv, S, Wn, lens, bound = 2, 4, 256, [20, 37, 300], 512
    B = len(lens)
    say(f"NaN rows past the length: {dt} d={d} lens={lens} bound={bound}")
    K, V = logical_kv(81, B, Hkv, d, max(lens) + 8, tdtype(dt))
    cache = W.KVCache.contiguous(B, Hkv, d, bound + 8, tdtype(dt))
    append_each(cache, K, V, [0] * B, lens)
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt))
    append_each(ring, K, V, [0] * B, lens)
    slack = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt), slack=3)  # the masked-ring kernels
    append_each(slack, K, V, [0] * B, lens)
    kn = torch.stack([K[b, :, lens[b]:lens[b] + 6].permute(1, 0, 2) for b in range(B)]).contiguous()
    vn = torch.stack([V[b, :, lens[b]:lens[b] + 6].permute(1, 0, 2) for b in range(B)]).contiguous()
    k1, v1 = kn[:, :1].contiguous(), vn[:, :1].contiguous()  # a draft step's token

    def attn(c, q, Hq, m, kind):
        o = torch.full((B, m, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        l = torch.full((B, m, Hq), float("nan"), dtype=torch.float32, device=DEV)
        if kind == "windowed":
            W.wmtp_draft_attn_windowed(c, q, Hq, 0.1, o, l, W.workspace(B, Hq, Hkv, d, 1, c.capacity))
        elif kind == "full":
            W.wmtp_draft_attn_full(c, q, Hq, 0.1, bound, o, l, W.workspace(B, Hq, Hkv, d, 1, bound))
        elif kind == "verify":
            W.wmtp_verify_attn(c, q, m, Hq, 0.1, bound, o, l, W.workspace(B, Hq, Hkv, d, m, bound))
        elif kind == "step_windowed":
            W.wmtp_draft_step_windowed(c, k1, v1, q, Hq, 0.1, o, l,
                                       W.workspace(B, Hq, Hkv, d, 1, c.capacity))
        elif kind == "step_full":
            W.wmtp_draft_step_full(c, k1, v1, q, Hq, 0.1, bound, o, l,
                                   W.workspace(B, Hq, Hkv, d, 1, bound))
        else:  # verify_step
            W.wmtp_verify_step(c, kn[:, :m].contiguous(), vn[:, :m].contiguous(), q, m, Hq, 0.1,
                               bound, o, l, W.workspace(B, Hq, Hkv, d, m, bound))
        return o, l

    # G = 4 and 16 (key-split kernel), G = 32 or G = 16 with m = 4 (32 and 64 rows: cooperative
    # kernel where it runs), G = 8 with m = 3, 4, 6 (verification in 24, 32 and 48 rows: the
    # key-split kernel with two and three row blocks where they fit its row limit)
    cases = [(8, 1, "windowed", ring), (8, 1, "full", cache), (8, 1, "step_windowed", ring),
             (8, 1, "step_full", cache), (8, 4, "verify", cache), (32, 4, "verify", cache),
             (16, 3, "verify", cache), (16, 4, "verify", cache), (16, 6, "verify", cache),
             (16, 4, "verify_step", cache),
             (32, 4, "verify_step", cache), (32, 1, "windowed", ring), (32, 1, "full", cache),
             (8, 1, "windowed", slack), (8, 1, "step_windowed", slack), (64, 1, "windowed", ring),
             (64, 1, "windowed", slack)]
    for Hq, m, kind, base in cases:
        q = synth.queries(82, m, B, m, Hq, d, tdtype(dt), DEV)
        clean = W.KVCache(base.k.clone(), base.v.clone(),
                          None if base.pos is None else base.pos.clone(), base.seq_len.clone(),
                          B, Hkv, d, base.capacity, base.sink, base.window, base.dtype)
        dirty = _poison(base, lens)
        o1, l1 = attn(clean, q, Hq, m, kind)
        o2, l2 = attn(dirty, q, Hq, m, kind)
        assert torch.isfinite(o1).all(), f"{kind} Hq={Hq} m={m}: non-finite output"
        assert torch.equal(o1, o2) and torch.equal(l1, l2), \
            f"{kind} Hq={Hq} m={m}: rows past the length changed the results"

    # MASW step: ring (past each length) and memory-slot cache (past each slot count) both poisoned
    counts, max_slots = [5, 9, 0], 64
    Ks, Vs = logical_kv(83, B, Hkv, d, max(counts), tdtype(dt))
    slots = W.KVCache.contiguous(B, Hkv, d, max_slots, tdtype(dt))
    append_each(slots, Ks, Vs, [0] * B, counts)
    for Hq, rb in ((8, ring), (8, slack), (64, ring)):
        q = synth.queries(84, 0, B, 1, Hq, d, tdtype(dt), DEV)
        res = []
        for r_, s_ in ((rb, slots), (_poison(rb, lens), _poison(slots, counts))):
            o = torch.full((B, 1, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
            l = torch.full((B, 1, Hq), float("nan"), dtype=torch.float32, device=DEV)
            W.wmtp_draft_attn_masw(r_, s_, q, Hq, 0.1, max_slots, o, l,
                                   W.masw_workspace(B, Hq, Hkv, d, r_.capacity, max_slots))
            res.append((o, l))
        assert torch.isfinite(res[0][0]).all(), f"masw Hq={Hq}: non-finite output"
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), \
            f"masw Hq={Hq}: rows past the lengths changed the results"


# ------------------------------------------------------------------------------------------
# a NaN INSIDE the attended set reaches the results (as in exact arithmetic): the merge must not
# drop the partial that holds it and keep a finite, wrong result built from the other partials
# ------------------------------------------------------------------------------------------
def _compare_nan(out, lse, ref_out, ref_lse, dt, what):
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.array_equal(np.isnan(o), np.isnan(ref_out)), f"{what}: NaN outputs differ"
    assert np.array_equal(np.isnan(l), np.isnan(ref_lse)), f"{what}: NaN lse differ"
    assert np.isnan(ref_out).any(), f"{what}: the planted NaN did not reach the oracle"
    ok = ~np.isnan(ref_out)
    err = float(np.max(np.abs(o[ok] - ref_out[ok])))
    okl = np.isfinite(ref_lse)
    lerr = float(np.max(np.abs(l[okl] - ref_lse[okl])))
    say(f"  {what}: NaN pattern equal; elsewhere max|out-ref| = {err:.3e} lse {lerr:.3e}")
    assert err <= TOL[dt] and lerr <= TOL[dt], what


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 256), ("f32", 64)])
def test_nan_inside_the_attended_set_propagates(dt, d):
    """One K row (sequence 0, KV head 0) and one V element (sequence 1, KV head 1) hold NaN at
    attended positions: exactly the outputs the oracle makes NaN are NaN (the whole query group
    for the K row, one dimension for the V element), on the key-split kernel (windowed ring, full
    draft, verification in 8 and 32 rows per KV head) and the cooperative kernel (draft reads of a
    32-head group, verification in 64 rows)."""
    B, Hkv, S, Wn, n, bound = 2, 2, 4, 64, 700, 1024
    say(f"NaN inside the attended set: {dt} d={d}")
    K, V = logical_kv(85, B, Hkv, d, n, tdtype(dt))
    K[0, 0, n - 3] = float("nan")           # a window position (also seen by the full read)
    V[1, 1, n - 10, d // 2 + 1] = float("nan")
    kv = oracle_kv(K, V, dt)
    cache = W.KVCache.contiguous(B, Hkv, d, bound, tdtype(dt))
    append_each(cache, K, V, [0] * B, [n] * B)
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, tdtype(dt))
    append_each(ring, K, V, [0] * B, [n] * B)
    scale = 1.0 / math.sqrt(d)
    for Hq in (16, 64):
        q = synth.queries(86, Hq, B, 1, Hq, d, tdtype(dt), DEV)
        qh = synth.host_array(q)
        o, l = run_windowed(ring, q, Hq, scale)
        ro, rl = oracle.draft_windowed(qh, ocode(dt), kv, [n] * B, S, Wn, scale)
        _compare_nan(o, l, ro, rl, dt, f"windowed Hq={Hq}")
        o, l = run_full(cache, q, Hq, scale, bound)
        ro, rl = oracle.draft_full(qh, ocode(dt), kv, [n] * B, scale)
        _compare_nan(o, l, ro, rl, dt, f"full Hq={Hq}")
    for Hq, m in ((16, 4), (8, 2), (32, 4)):
        q = synth.queries(87, m, B, m, Hq, d, tdtype(dt), DEV)
        o, l = run_verify(cache, q, Hq, scale, bound)
        ro, rl = oracle.verify(synth.host_array(q), ocode(dt), kv, [n] * B, scale)
        _compare_nan(o, l, ro, rl, dt, f"verify Hq={Hq} m={m}")
