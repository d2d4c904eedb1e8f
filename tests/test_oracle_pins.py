"""Pins of the float64 oracle to things other than itself (CPU only).

Each test ties the oracle to the mathematics of softmax attention, to an independent library
routine (torch's scaled_dot_product_attention / logsumexp in float64), to brute force on tiny
inputs, to closed forms, or to the figure the Windowed-MTP abstract prints. Together they are
chosen so that a dropped term, an off-by-one in the sink/window/causal sets, a transposed operand,
a wrong GQA mapping, a wrong bf16 decode or a wrong ring slot map each fail at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F32, F64

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, masks, scale):
    """torch float64 reference. q [B][m][Hq][d]; k,v [B][Hkv][n][d]; masks [B][m][n] bool."""
    B, m, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)  # B Hq m d
    tk = torch.from_numpy(k).repeat_interleave(G, dim=1)  # B Hq n d  (head hq reads hq // G)
    tv = torch.from_numpy(v).repeat_interleave(G, dim=1)
    tm = torch.from_numpy(masks)[:, None, :, :].expand(B, Hq, m, k.shape[2])
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    logits = (tq @ tk.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~tm, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def _mask_from_filter(B, m, n_total, keep):
    masks = np.zeros((B, m, n_total), dtype=bool)
    for b in range(B):
        for j in range(m):
            for p in range(n_total):
                masks[b, j, p] = keep(b, j, p)
    return masks


# ------------------------------------------------------------------------------------------
# P4: independent library routine (torch SDPA + logsumexp, float64)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,d,n", [(1, 8, 2, 16, 37), (2, 6, 3, 8, 20), (3, 4, 4, 5, 9)])
def test_full_matches_torch_sdpa(oracle_lib, B, Hq, Hkv, d, n):
    q = _rand((B, 1, Hq, d), 1)
    k = _rand((B, Hkv, n, d), 2)
    v = _rand((B, Hkv, n, d), 3)
    lens = [n - b for b in range(B)]  # ragged: sequence b holds n - b tokens
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.draft_full(q, F64, oracle.contiguous_kv(k, v, F64), lens, scale)
    masks = _mask_from_filter(B, 1, n, lambda b, j, p: p < lens[b])
    ro, rl = _sdpa(q, k, v, masks, scale)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,W,n", [(4, 8, 30), (0, 5, 17), (2, 1, 9), (3, 16, 12), (1, 3, 4)])
def test_windowed_matches_torch_sdpa(oracle_lib, S, W, n):
    B, Hq, Hkv, d = 2, 4, 2, 8
    q = _rand((B, 1, Hq, d), 4)
    k = _rand((B, Hkv, n, d), 5)
    v = _rand((B, Hkv, n, d), 6)
    lens = [n, n - 1]
    out, lse = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k, v, F64), lens, S, W, 0.4)
    # sinks: the first S positions; window: the last W of the tokens present
    masks = _mask_from_filter(B, 1, n, lambda b, j, p: p < lens[b] and (p < S or p >= lens[b] - W))
    ro, rl = _sdpa(q, k, v, masks, 0.4)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_verify_matches_torch_sdpa(oracle_lib, m):
    B, Hq, Hkv, d, n = 2, 8, 2, 16, 25
    q = _rand((B, m, Hq, d), 7)
    k = _rand((B, Hkv, n, d), 8)
    v = _rand((B, Hkv, n, d), 9)
    lens = [n, n - 3]
    out, lse = oracle.verify(q, F64, oracle.contiguous_kv(k, v, F64), lens, 0.25)
    # candidate j sits at position lens-m+j and sees everything up to itself
    masks = _mask_from_filter(B, m, n, lambda b, j, p: p <= lens[b] - m + j)
    ro, rl = _sdpa(q, k, v, masks, 0.25)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_bf16_and_f32_inputs_decode_exactly(oracle_lib):
    """bf16 bit patterns and float32 inputs must give the float64 result of their exact values
    (torch's own bf16 -> float64 widening is the reference)."""
    B, Hq, Hkv, d, n = 1, 4, 1, 32, 40
    g = torch.Generator().manual_seed(11)
    qb = torch.randn(B, 1, Hq, d, generator=g).to(torch.bfloat16)
    kb = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16)
    vb = torch.randn(B, Hkv, n, d, generator=g).to(torch.bfloat16)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    out_b, lse_b = oracle.draft_full(bits(qb), BF16, oracle.contiguous_kv(bits(kb), bits(vb), BF16),
                                     [n], 0.2)
    out_d, lse_d = oracle.draft_full(qb.double().numpy(), F64,
                                     oracle.contiguous_kv(kb.double().numpy(), vb.double().numpy(),
                                                          F64), [n], 0.2)
    assert np.array_equal(out_b, out_d) and np.array_equal(lse_b, lse_d)
    qf, kf, vf = qb.float(), kb.float(), vb.float()
    out_f, _ = oracle.draft_full(qf.numpy(), F32, oracle.contiguous_kv(kf.numpy(), vf.numpy(), F32),
                                 [n], 0.2)
    assert np.array_equal(out_f, out_d)
    masks = np.ones((B, 1, n), dtype=bool)
    ro, rl = _sdpa(qb.double().numpy(), kb.double().numpy(), vb.double().numpy(), masks, 0.2)
    np.testing.assert_allclose(out_b, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_b, rl, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------
# P5: brute force on tiny inputs (pure Python, math.exp + math.fsum)
# ------------------------------------------------------------------------------------------
def _brute(qv, krows, vrows, scale):
    s = [scale * math.fsum(a * b for a, b in zip(qv, kr)) for kr in krows]
    M = max(s)
    w = [math.exp(x - M) for x in s]
    Z = math.fsum(w)
    o = [math.fsum(w[p] * vrows[p][i] for p in range(len(w))) / Z for i in range(len(qv))]
    return o, M + math.log(Z)


@pytest.mark.parametrize("n,S,W", [(1, 2, 3), (5, 1, 2), (12, 2, 4), (16, 0, 16), (16, 3, 5)])
def test_brute_force_tiny(oracle_lib, n, S, W):
    d, Hq, Hkv = 6, 2, 1
    q = _rand((1, 1, Hq, d), 20)
    k = _rand((1, Hkv, n, d), 21)
    v = _rand((1, Hkv, n, d), 22)
    kv = oracle.contiguous_kv(k, v, F64)
    of, lf = oracle.draft_full(q, F64, kv, [n], 0.7)
    ow, lw = oracle.draft_windowed(q, F64, kv, [n], S, W, 0.7)
    for hq in range(Hq):
        full_set = list(range(n))
        win_set = [p for p in range(n) if p < S or p >= n - W]
        for out, lse, chosen in ((of, lf, full_set), (ow, lw, win_set)):
            o_ref, l_ref = _brute(q[0, 0, hq], [k[0, 0, p] for p in chosen],
                                  [v[0, 0, p] for p in chosen], 0.7)
            np.testing.assert_allclose(out[0, 0, hq], o_ref, rtol=0, atol=1e-14)
            assert abs(lse[0, 0, hq] - l_ref) < 1e-13


# ------------------------------------------------------------------------------------------
# P6: closed forms and special cases
# ------------------------------------------------------------------------------------------
def test_equal_keys_give_mean_of_values_and_log_count(oracle_lib):
    n, d, S, W = 40, 8, 3, 10
    q = _rand((1, 1, 2, d), 30)
    k = np.tile(_rand((1, 1, 1, d), 31), (1, 1, n, 1))
    v = _rand((1, 1, n, d), 32)
    kv = oracle.contiguous_kv(k, v, F64)
    s = 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])
    o, l = oracle.draft_windowed(q, F64, kv, [n], S, W, 0.5)
    # attended: positions 0,1,2 and 30..39 -> 13 positions
    expect = (v[0, 0, :3].sum(0) + v[0, 0, 30:].sum(0)) / 13.0
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=0, atol=1e-13)
    assert abs(l[0, 0, 0] - (s + math.log(13))) < 1e-12


def test_zero_query_gives_uniform_weights(oracle_lib):
    n, d, m = 17, 4, 3
    q = np.zeros((1, m, 2, d))
    k = _rand((1, 1, n, d), 33)
    v = _rand((1, 1, n, d), 34)
    o, l = oracle.verify(q, F64, oracle.contiguous_kv(k, v, F64), [n], 1.0)
    for j in range(m):
        visible = n - m + j + 1  # candidates at 14,15,16; candidate j sees 0..14+j
        np.testing.assert_allclose(o[0, j, 1], v[0, 0, :visible].mean(0), rtol=0, atol=1e-14)
        assert abs(l[0, j, 1] - math.log(visible)) < 1e-14


def test_constant_values_give_that_constant(oracle_lib):
    n, d = 23, 5
    q = _rand((1, 1, 3, d), 35)
    k = _rand((1, 1, n, d), 36)
    c = _rand((d,), 37)
    v = np.tile(c, (1, 1, n, 1))
    o, _ = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k, v, F64), [n], 2, 6, 1.0)
    np.testing.assert_allclose(o[0, 0], np.tile(c, (3, 1)), rtol=0, atol=1e-14)


def test_window_of_one_without_sinks_returns_last_value(oracle_lib):
    """S = 0, W = 1: the draft sees only the newest token, so o = v_{n-1} exactly."""
    n, d = 19, 6
    q = _rand((1, 1, 2, d), 38)
    k = _rand((1, 1, n, d), 39)
    v = _rand((1, 1, n, d), 40)
    o, l = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k, v, F64), [n], 0, 1, 0.3)
    assert np.array_equal(o[0, 0, 0], v[0, 0, n - 1])
    assert abs(l[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, n - 1])) < 1e-14


def test_one_sink_one_window_is_two_way_softmax(oracle_lib):
    n, d = 11, 4
    q = _rand((1, 1, 1, d), 41)
    k = _rand((1, 1, n, d), 42)
    v = _rand((1, 1, n, d), 43)
    o, _ = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k, v, F64), [n], 1, 1, 1.0)
    s0, s1 = float(q[0, 0, 0] @ k[0, 0, 0]), float(q[0, 0, 0] @ k[0, 0, n - 1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(o[0, 0, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, n - 1], atol=1e-14)


def _spike(n, d, hot, seed):
    """Keys such that the query has a logit 100 above every other key at position `hot`."""
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = _rand((1, 1, n, d), seed) * 0.01
    k[0, 0, hot, 0] = 100.0
    v = _rand((1, 1, n, d), seed + 1)
    return q, k, v


def test_spike_at_first_dropped_position(oracle_lib):
    """n = S + W + 1: exactly position S leaves the attended set. A dominant key there decides
    the full result and is invisible to the windowed one."""
    S, W, d = 4, 8, 4
    n = S + W + 1
    q, k, v = _spike(n, d, S, 44)
    kv = oracle.contiguous_kv(k, v, F64)
    of, _ = oracle.draft_full(q, F64, kv, [n], 1.0)
    ow, _ = oracle.draft_windowed(q, F64, kv, [n], S, W, 1.0)
    np.testing.assert_allclose(of[0, 0, 0], v[0, 0, S], atol=n * math.exp(-99))
    assert np.abs(ow[0, 0, 0] - v[0, 0, S]).max() > 0.1
    # the neighbours of the dropped position stay visible
    for hot in (S - 1, S + 1, n - 1):
        q2, k2, v2 = _spike(n, d, hot, 45)
        ow2, _ = oracle.draft_windowed(q2, F64, oracle.contiguous_kv(k2, v2, F64), [n], S, W, 1.0)
        np.testing.assert_allclose(ow2[0, 0, 0], v2[0, 0, hot], atol=n * math.exp(-99))


def test_spike_at_causal_boundary(oracle_lib):
    """Verify: candidate j sees position n-m+j and not n-m+j+1."""
    n, m, d = 30, 4, 4
    for j in range(m - 1):
        q1, k1, v1 = _spike(n, d, n - m + j, 46)
        q1 = np.repeat(q1, m, axis=1)
        o1, _ = oracle.verify(q1, F64, oracle.contiguous_kv(k1, v1, F64), [n], 1.0)
        np.testing.assert_allclose(o1[0, j, 0], v1[0, 0, n - m + j], atol=n * math.exp(-99))
        q2, k2, v2 = _spike(n, d, n - m + j + 1, 47)
        q2 = np.repeat(q2, m, axis=1)
        o2, _ = oracle.verify(q2, F64, oracle.contiguous_kv(k2, v2, F64), [n], 1.0)
        assert np.abs(o2[0, j, 0] - v2[0, 0, n - m + j + 1]).max() > 0.1


def test_empty_set_reading(oracle_lib):
    q = np.ones((1, 1, 1, 4))
    k = np.ones((1, 1, 4, 4))
    o, l = oracle.draft_full(q, F64, oracle.contiguous_kv(k, k, F64), [0], 1.0)
    assert np.all(o == 0) and l[0, 0, 0] == -np.inf


# ------------------------------------------------------------------------------------------
# P1: windowed equals full when the window covers everything
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 3, 4, 5, 100, 259, 260])
def test_windowed_equals_full_when_window_covers_all(oracle_lib, n):
    S, W, d = 4, 256, 16
    q = _rand((1, 1, 8, d), 50)
    k = _rand((1, 2, n, d), 51)
    v = _rand((1, 2, n, d), 52)
    kv = oracle.contiguous_kv(k, v, F64)
    of, lf = oracle.draft_full(q, F64, kv, [n], 0.25)
    ow, lw = oracle.draft_windowed(q, F64, kv, [n], S, W, 0.25)
    assert np.array_equal(of, ow) and np.array_equal(lf, lw)


def test_windowed_differs_from_full_past_the_window(oracle_lib):
    S, W, d = 4, 256, 16
    n = S + W + 1
    q = _rand((1, 1, 8, d), 53)
    k = _rand((1, 2, n, d), 54)
    v = _rand((1, 2, n, d), 55)
    kv = oracle.contiguous_kv(k, v, F64)
    of, _ = oracle.draft_full(q, F64, kv, [n], 0.25)
    ow, _ = oracle.draft_windowed(q, F64, kv, [n], S, W, 0.25)
    assert not np.array_equal(of, ow)


# ------------------------------------------------------------------------------------------
# P7: partition / log-sum-exp merge identity
# ------------------------------------------------------------------------------------------
def test_partition_merge_identity(oracle_lib):
    n, d = 64, 8
    q = _rand((1, 1, 4, d), 60)
    k = _rand((1, 2, n, d), 61)
    v = _rand((1, 2, n, d), 62)
    kv = oracle.contiguous_kv(k, v, F64)
    whole, lw = oracle.attention(q, F64, kv, [[[(0, n)]]], 0.3)
    a, la = oracle.attention(q, F64, kv, [[[(0, 13), (40, 50)]]], 0.3)
    b, lb = oracle.attention(q, F64, kv, [[[(13, 40), (50, n)]]], 0.3)
    lse = np.logaddexp(la, lb)
    merged = (np.exp(la - lse)[..., None] * a + np.exp(lb - lse)[..., None] * b)
    np.testing.assert_allclose(merged, whole, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lw, rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------------
# P3: invariance to the order of the attended rows
# ------------------------------------------------------------------------------------------
def test_permutation_invariance(oracle_lib):
    n, d, S, W = 50, 8, 3, 12
    q = _rand((1, 1, 4, d), 70)
    k = _rand((1, 2, n, d), 71)
    v = _rand((1, 2, n, d), 72)
    attended = [p for p in range(n) if p < S or p >= n - W]
    perm = np.random.default_rng(73).permutation(attended)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, attended] = k[:, :, perm]
    v2[:, :, attended] = v[:, :, perm]
    o1, l1 = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k, v, F64), [n], S, W, 0.3)
    o2, l2 = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k2, v2, F64), [n], S, W, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # a permutation that moves an unattended row into the set must change the result
    k3, v3 = k.copy(), v.copy()
    k3[:, :, [S, n - 1]] = k[:, :, [n - 1, S]]
    v3[:, :, [S, n - 1]] = v[:, :, [n - 1, S]]
    o3, _ = oracle.draft_windowed(q, F64, oracle.contiguous_kv(k3, v3, F64), [n], S, W, 0.3)
    assert np.abs(o3 - o1).max() > 1e-6


# ------------------------------------------------------------------------------------------
# P9 + ring conventions: the compact ring buffer
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("S,W", [(4, 8), (0, 5), (1, 1), (3, 16)])
def test_ring_model_holds_sinks_and_last_window(S, W):
    model = oracle.RingModel(1, S, W)
    n = 0
    for step in [1, 2, 1, W + 3, 1, 7, 3 * (S + W) + 5, 1]:
        model.append(0, step)
        n += step
        occ = model.occupied_slots(0)
        held = sorted(model.tags[0, occ].tolist())
        expect = list(range(min(S, n))) + list(range(max(S, n - W), n))
        assert held == expect
        assert len(occ) == min(n, S + W)
        assert occ.tolist() == list(range(min(n, S + W)))  # occupied slots are a prefix
        for s in occ:
            assert oracle.ring_slot(int(model.tags[0, s]), S, W) == s


def test_ring_slot_convention():
    """Reading: the first window token lands in slot S; then the window wraps over W slots."""
    S, W = 4, 8
    assert [oracle.ring_slot(p, S, W) for p in range(S)] == list(range(S))
    assert oracle.ring_slot(S, S, W) == S
    assert oracle.ring_slot(S + W - 1, S, W) == S + W - 1
    assert oracle.ring_slot(S + W, S, W) == S
    p = np.arange(0, 100)
    assert np.array_equal(oracle.ring_slot(p, S, W),
                          np.array([oracle.ring_slot(int(x), S, W) for x in p]))
    assert oracle.ring_slot(12345, 77, 0) == 12345  # contiguous cache: the identity map


def test_ring_model_bulk_equals_token_by_token():
    S, W = 3, 5
    a = oracle.RingModel(1, S, W)
    b = oracle.RingModel(1, S, W)
    a.append(0, 37)
    for _ in range(37):
        b.append(0, 1)
    assert np.array_equal(a.tags, b.tags)


# ------------------------------------------------------------------------------------------
# P2: attention over the ring layout equals attention over the masked logical sequence
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n", [5, 12, 13, 40, 97])
def test_ring_layout_equals_masked_sequence(oracle_lib, n):
    S, W, d, Hq, Hkv = 4, 8, 8, 4, 2
    q = _rand((1, 1, Hq, d), 80)
    k = _rand((1, Hkv, n, d), 81)
    v = _rand((1, Hkv, n, d), 82)
    kv = oracle.contiguous_kv(k, v, F64)
    model = oracle.RingModel(1, S, W)
    model.append(0, n)
    rk, rv = oracle.ring_expected(model, kv)
    o_ring, l_ring = oracle.ring_attention(q, F64, rk, rv, F64, model.tags, 0.3)
    o_seq, l_seq = oracle.draft_windowed(q, F64, kv, [n], S, W, 0.3)
    np.testing.assert_allclose(o_ring, o_seq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_ring, l_seq, rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------------
# P8: verification reduces to the draft forms
# ------------------------------------------------------------------------------------------
def test_verify_single_candidate_is_full_draft(oracle_lib):
    n, d = 33, 8
    q = _rand((2, 1, 4, d), 90)
    k = _rand((2, 2, n, d), 91)
    v = _rand((2, 2, n, d), 92)
    kv = oracle.contiguous_kv(k, v, F64)
    ov, lv = oracle.verify(q, F64, kv, [n, n - 4], 0.3)
    of, lf = oracle.draft_full(q, F64, kv, [n, n - 4], 0.3)
    assert np.array_equal(ov, of) and np.array_equal(lv, lf)


def test_verify_row_is_full_draft_on_its_prefix(oracle_lib):
    n, d, m = 33, 8, 4
    q = _rand((1, m, 4, d), 93)
    k = _rand((1, 2, n, d), 94)
    v = _rand((1, 2, n, d), 95)
    kv = oracle.contiguous_kv(k, v, F64)
    ov, lv = oracle.verify(q, F64, kv, [n], 0.3)
    for j in range(m):
        of, lf = oracle.draft_full(q[:, j:j + 1], F64, kv, [n - m + j + 1], 0.3)
        assert np.array_equal(ov[:, j:j + 1], of) and np.array_equal(lv[:, j:j + 1], lf)


# ------------------------------------------------------------------------------------------
# P10: the figure the pages print
# ------------------------------------------------------------------------------------------
def test_dropped_fraction_matches_page_figure():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        fig = json.load(f)["dropped_fraction_at_1M"]
    n = fig["context_tokens"] + 1  # one draft token appended to a 1M prefix
    dropped = oracle.dropped_fraction(n, 4, 4096)
    assert abs(dropped - fig["value"]) <= 0.01  # "about 99%"
    # the kept set is a constant: it does not grow with the context
    for ctx in (1 << 17, 1 << 19, 1 << 20, 1 << 21):
        kept = sum(b - a for a, b in oracle.windowed_positions(ctx, 4, 4096))
        assert kept == 4100


# ------------------------------------------------------------------------------------------
# Ring rollback (MASW page, section 4.3: speculative local KV is discarded after a rejection)
# ------------------------------------------------------------------------------------------
def _attended_positions(model, b=0):
    return sorted(model.tags[b, model.attended_slots(b)].tolist())


@pytest.mark.parametrize("S,W,slack", [(4, 8, 3), (0, 5, 5), (1, 1, 2), (3, 16, 4)])
def test_rollback_returns_to_the_state_without_the_rejected_tokens(S, W, slack):
    """After any interleaving of appends and rollbacks (each at most `slack` deep), the attended
    positions are exactly the sinks and the last W of the n present, at their slot-map slots, and
    they sit where a ring that appended only those n tokens holds them."""
    rng = np.random.default_rng(S * 100 + W * 10 + slack)
    model = oracle.RingModel(1, S, W, slack)
    n = 0
    for step in range(60):
        c = int(rng.integers(1, slack + 3))
        model.append(0, c)
        n += c
        d = int(rng.integers(0, c + 1))
        got = model.rollback(0, d)
        assert got == min(d, slack, n)
        n -= got
        assert model.n[0] == n
        expect = list(range(min(S, n))) + list(range(max(S, n - W), n))
        assert _attended_positions(model) == expect
        fresh = oracle.RingModel(1, S, W, slack)
        fresh.append(0, n)
        slots = model.attended_slots(0)
        assert np.array_equal(slots, fresh.attended_slots(0))
        assert np.array_equal(model.tags[0, slots], fresh.tags[0, slots])
        for s in slots:
            assert oracle.ring_slot(int(model.tags[0, s]), S, W + slack) == s


def test_rollback_is_clamped_to_the_slack_and_marks_slots_empty():
    model = oracle.RingModel(1, 2, 4, 2)
    model.append(0, 10)
    before = model.tags.copy()
    assert model.rollback(0, 5) == 2  # only the slack can be undone exactly
    assert model.n[0] == 8
    # slots of positions 8 and 9 are now empty; every other slot is unchanged
    emptied = [oracle.ring_slot(p, 2, 6) for p in (8, 9)]
    assert all(model.tags[0, s] == -1 for s in emptied)
    keep = [s for s in range(8) if s not in emptied]
    assert np.array_equal(model.tags[0, keep], before[0, keep])
    assert model.rollback(0, -3) == 0
    none = oracle.RingModel(1, 2, 4, 0)
    none.append(0, 10)
    assert none.rollback(0, 1) == 0  # a compact ring without slack cannot roll back
    flat = oracle.RingModel(1, 64, 0, 0)  # contiguous cache: nothing is overwritten
    flat.append(0, 10)
    assert flat.rollback(0, 7) == 7 and flat.n[0] == 3
    assert flat.tags[0, :3].tolist() == [0, 1, 2] and (flat.tags[0, 3:] == -1).all()


def test_second_rollback_stops_where_the_window_was_overwritten():
    """A rollback deeper than what was appended since the previous one: with W = 7 and slack = 3
    after 19 appends, append 1 and discard 3 (n = 17), then append 1 and ask for 3 again. The
    first append wrote position 19 over position 9 and the second wrote position 17 back into its
    own slot, so n may only go back to 17 (the window 10..16 is held; 8..9 are not): the second
    rollback discards 1 token, not 3."""
    for S in (0, 2):
        model = oracle.RingModel(1, S, 7, 3)
        model.append(0, 19)
        model.append(0, 1)
        assert model.rollback(0, 3) == 3 and model.n[0] == 17
        model.append(0, 1)
        assert model.rollback(0, 3) == 1 and model.n[0] == 17
        expect = list(range(min(S, 17))) + list(range(max(S, 10), 17))
        assert _attended_positions(model) == expect


def _replay_held(ops, S, W, slack):
    """Positions held after a log of ('append', count) / ('drop', d) operations, replayed token by
    token into a dict slot -> position (a slot keeps the last position written to it; a dropped
    position's slot is emptied)."""
    slots, n = {}, 0
    for op, c in ops:
        if op == "append":
            for p in range(n, n + c):
                slots[p if p < S else S + (p - S) % (W + slack)] = p
            n += c
        else:
            for p in range(n - c, n):
                slots.pop(p if p < S else S + (p - S) % (W + slack), None)
            n -= c
    return set(slots.values()), n


@pytest.mark.parametrize("S,W,slack", [(4, 8, 3), (0, 5, 5), (1, 1, 2), (3, 16, 9), (2, 3, 12)])
def test_rollback_depth_is_the_deepest_that_keeps_the_window(S, W, slack):
    """Rollbacks of any requested depth, deeper than the last append included: the depth the model
    takes is the largest d <= min(request, n, slack) for which every position of the remaining
    sinks + last-W set is held, where 'held' comes from replaying the whole operation log into a
    plain slot dictionary (no ring model)."""
    rng = np.random.default_rng(S * 1000 + W * 10 + slack + 1)
    model = oracle.RingModel(1, S, W, slack)
    ops = []
    for step in range(80):
        c = int(rng.integers(1, slack + 3))
        model.append(0, c)
        ops.append(("append", c))
        req = int(rng.integers(-1, slack + 4))
        held, n = _replay_held(ops, S, W, slack)

        def keeps(d):
            need = set(range(min(S, n - d))) | set(range(max(S, n - d - W), n - d))
            return need <= held

        cap = max(0, min(req, n, slack))
        want = max(d for d in range(cap + 1) if keeps(d))
        got = model.rollback(0, req)
        assert got == want, (step, n, req)
        ops.append(("drop", got))
        assert _attended_positions(model) == sorted(
            set(range(min(S, n - got))) | set(range(max(S, n - got - W), n - got)))


def test_rollback_then_reappend_attends_the_replacement_tokens(oracle_lib):
    """Speculative loop on real rows: drafts are appended, some rejected and replaced by other
    tokens at the same positions. Attention over the ring's attended slots equals windowed
    attention over the final logical sequence (the rows each position ends up holding)."""
    S, W, slack, Hkv, Hq, d = 3, 7, 4, 2, 4, 8
    rng = np.random.default_rng(7)
    model = oracle.RingModel(1, S, W, slack)
    nslots = S + W + slack
    ring_k = np.zeros((1, Hkv, nslots, d))
    ring_v = np.zeros((1, Hkv, nslots, d))
    seq_k, seq_v = [], []  # final content of every position, as lists of [Hkv][d] rows

    def write(rows_k, rows_v):
        for rk, rv in zip(rows_k, rows_v):
            p = int(model.n[0])
            s = oracle.ring_slot(p, S, W + slack)
            ring_k[0, :, s], ring_v[0, :, s] = rk, rv
            model.append(0, 1)
            if p < len(seq_k):
                seq_k[p], seq_v[p] = rk, rv
            else:
                seq_k.append(rk)
                seq_v.append(rv)

    write(rng.standard_normal((20, Hkv, d)), rng.standard_normal((20, Hkv, d)))
    for step in range(12):
        k = int(rng.integers(1, slack + 1))
        write(rng.standard_normal((k, Hkv, d)), rng.standard_normal((k, Hkv, d)))
        drop = model.rollback(0, int(rng.integers(0, k + 1)))
        del seq_k[len(seq_k) - drop:], seq_v[len(seq_v) - drop:]
        write(rng.standard_normal((1, Hkv, d)), rng.standard_normal((1, Hkv, d)))  # correction
        n = int(model.n[0])
        assert n == len(seq_k)
        q = rng.standard_normal((1, 1, Hq, d))
        lk = np.stack(seq_k, axis=1)[None]
        lv = np.stack(seq_v, axis=1)[None]
        o_seq, l_seq = oracle.draft_windowed(q, F64, oracle.contiguous_kv(lk, lv, F64), [n], S,
                                             W, 0.4)
        o_ring, l_ring = oracle.ring_attention(q, F64, ring_k, ring_v, F64, model.tags, 0.4,
                                               slots=[model.attended_slots(0)])
        np.testing.assert_allclose(o_ring, o_seq, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l_ring, l_seq, rtol=0, atol=1e-13)


# ------------------------------------------------------------------------------------------
# Greedy accept/reject (the target's standard rule under greedy decoding)
# ------------------------------------------------------------------------------------------
def test_greedy_accept_hand_cases():
    V = 6
    logits = np.full((3, 4, V), -1.0)
    choice = [[2, 5, 1, 0], [2, 5, 1, 0], [3, 3, 3, 4]]
    for b in range(3):
        for i in range(4):
            logits[b, i, choice[b][i]] = 2.0
    draft = np.array([[2, 5, 1], [2, 4, 1], [0, 3, 3]])
    ch, n_acc, nxt, drop = oracle.greedy_accept(logits, draft)
    assert ch.tolist() == choice
    assert n_acc.tolist() == [3, 1, 0]  # all kept; second rejected; first rejected
    assert nxt.tolist() == [0, 5, 3]  # bonus token; correction at row 1; correction at row 0
    assert drop.tolist() == [0, 2, 3]


def test_greedy_accept_ties_take_the_lowest_index():
    logits = np.zeros((1, 2, 5))
    logits[0, 0, [1, 3]] = 7.0
    logits[0, 1, [4, 0]] = 7.0
    ch, n_acc, nxt, _ = oracle.greedy_accept(logits, np.array([[3]]))
    assert ch.tolist() == [[1, 0]]
    assert n_acc.tolist() == [0] and nxt.tolist() == [1]
    ch, n_acc, nxt, _ = oracle.greedy_accept(logits, np.array([[1]]))
    assert n_acc.tolist() == [1] and nxt.tolist() == [0]


def test_greedy_accept_matches_plain_loops():
    """Brute force with Python loops and comparisons (no argmax routine)."""
    rng = np.random.default_rng(11)
    B, k, V = 5, 4, 9
    for trial in range(30):
        logits = rng.integers(-3, 4, size=(B, k + 1, V)).astype(np.float64)  # many ties
        draft = rng.integers(0, V, size=(B, k))
        ch, n_acc, nxt, drop = oracle.greedy_accept(logits, draft)
        for b in range(B):
            picks = []
            for i in range(k + 1):
                best = 0
                for t in range(1, V):
                    if logits[b, i, t] > logits[b, i, best]:
                        best = t
                picks.append(best)
            a = 0
            while a < k and draft[b, a] == picks[a]:
                a += 1
            assert ch[b].tolist() == picks
            assert n_acc[b] == a and nxt[b] == picks[a] and drop[b] == k - a


# ------------------------------------------------------------------------------------------
# MASW working memory: sinks + memory slots + local window (MASW page, section 4.1)
# ------------------------------------------------------------------------------------------
def _masw_case(seed, n, M, d=8, Hq=4, Hkv=2):
    q = _rand((1, 1, Hq, d), seed)
    k = _rand((1, Hkv, n, d), seed + 1)
    v = _rand((1, Hkv, n, d), seed + 2)
    sk = _rand((1, Hkv, M, d), seed + 3)
    sv = _rand((1, Hkv, M, d), seed + 4)
    return q, k, v, sk, sv


def test_masw_without_slots_is_the_windowed_draft(oracle_lib):
    q, k, v, sk, sv = _masw_case(90, 50, 6)
    kv = oracle.contiguous_kv(k, v, F64)
    o1, l1 = oracle.draft_masw(q, F64, kv, [50], 4, 8, sk, sv, [0], 0.3)
    o2, l2 = oracle.draft_windowed(q, F64, kv, [50], 4, 8, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("n,S,W,m", [(50, 4, 8, 6), (9, 4, 8, 3), (40, 0, 5, 1), (3, 4, 8, 5)])
def test_masw_matches_torch_sdpa_over_the_union(oracle_lib, n, S, W, m):
    """P4-style pin: torch SDPA (float64) over the explicitly concatenated working set."""
    q, k, v, sk, sv = _masw_case(100 + n, n, 6)
    kv = oracle.contiguous_kv(k, v, F64)
    o, l = oracle.draft_masw(q, F64, kv, [n], S, W, sk, sv, [m], 0.35)
    keep = [p for p in range(n) if p < S or p >= n - W]
    kk = np.concatenate([k[:, :, keep], sk[:, :, :m]], axis=2)
    vv = np.concatenate([v[:, :, keep], sv[:, :, :m]], axis=2)
    masks = np.ones((1, 1, kk.shape[2]), dtype=bool)
    ro, rl = _sdpa(q, kk, vv, masks, 0.35)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-12)


def test_masw_is_the_lse_merge_of_window_and_slots(oracle_lib):
    """Partition identity: the union's result is the log-sum-exp merge of the windowed part and
    the slots-only part."""
    q, k, v, sk, sv = _masw_case(130, 60, 7)
    kv = oracle.contiguous_kv(k, v, F64)
    o, l = oracle.draft_masw(q, F64, kv, [60], 4, 8, sk, sv, [7], 0.3)
    ow, lw = oracle.draft_windowed(q, F64, kv, [60], 4, 8, 0.3)
    slots_only = oracle.contiguous_kv(sk, sv, F64)
    os_, ls = oracle.draft_full(q, F64, slots_only, [7], 0.3)
    L = np.logaddexp(lw, ls)
    merged = ow * np.exp(lw - L)[..., None] + os_ * np.exp(ls - L)[..., None]
    np.testing.assert_allclose(o, merged, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, L, rtol=0, atol=1e-13)


def test_masw_spike_in_a_slot_returns_that_slot(oracle_lib):
    q, k, v, sk, sv = _masw_case(140, 30, 5, d=4, Hq=2, Hkv=1)
    q[:] = 1.0
    sk[0, 0, 3] = 60.0  # one slot key scores 240 x scale above the rest
    kv = oracle.contiguous_kv(k, v, F64)
    o, _ = oracle.draft_masw(q, F64, kv, [30], 2, 6, sk, sv, [5], 1.0)
    np.testing.assert_allclose(o[0, 0, 0], sv[0, 0, 3], rtol=0, atol=1e-12)
