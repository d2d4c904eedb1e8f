"""A plain C program calls libwmtp.so (tests/c_caller/wmtp_c_caller.c: HIP runtime memory, no
torch, no Python): its ring bytes, position tags, lengths and attention outputs (windowed and
full draft reads, the target's append + verification of 8 candidates and a verification of the
last 3 positions, an allocation-free draft step on a ring with slack, greedy accept, the rollback
by the device's count, and a MASW-style read) match the host ring model, the greedy rule and the
float64 oracle on the same inputs, which the program writes out."""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_common import TOL, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_caller", "wmtp_c_caller")
HKV, G, D, S, W, N, MV, MV3 = 2, 4, 128, 4, 64, 300, 8, 3  # the program's shapes
SLACK, K_ACC, VOCAB, NSLOT = 4, 2, 1000, 37
NV, NV_CAP = N + MV, N + MV + 5  # verification cache: length after the step, capacity
HQ = HKV * G


def _load(d, name, dtype, shape):
    return np.fromfile(os.path.join(d, name), dtype=dtype).reshape(shape)


def test_c_program_calls_the_library(tmp_path):
    if not os.path.exists(EXE):  # normally built by the package build, beside its source
        from c_caller import build as c_build

        c_build.build()
    say("C caller: windowed, full and verification calls from a C program")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    d = str(tmp_path)
    kn = _load(d, "k_new.bin", np.uint16, (N, HKV, D))  # bf16 bits, token-major
    vn = _load(d, "v_new.bin", np.uint16, (N, HKV, D))
    q = _load(d, "q.bin", np.uint16, (1, 1, HQ, D))
    K = np.ascontiguousarray(kn.transpose(1, 0, 2))[None]  # [1][HKV][N][D]
    V = np.ascontiguousarray(vn.transpose(1, 0, 2))[None]
    kv = oracle.contiguous_kv(K, V, oracle.BF16)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    checks = (("windowed", oracle.draft_windowed(q, oracle.BF16, kv, [N], S, W, scale)),
              ("full", oracle.draft_full(q, oracle.BF16, kv, [N], scale)))
    # verification cache: the N prefix tokens then the MV candidates, position-major
    kc = _load(d, "k_cand.bin", np.uint16, (MV, HKV, D))
    vc = _load(d, "v_cand.bin", np.uint16, (MV, HKV, D))
    KV_ = np.concatenate([K, np.ascontiguousarray(kc.transpose(1, 0, 2))[None]], axis=2)
    VV_ = np.concatenate([V, np.ascontiguousarray(vc.transpose(1, 0, 2))[None]], axis=2)
    kv_v = oracle.contiguous_kv(KV_, VV_, oracle.BF16)
    qv = _load(d, "q_verify.bin", np.uint16, (1, MV, HQ, D))
    qv3 = _load(d, "q_verify3.bin", np.uint16, (1, MV3, HQ, D))
    checks += (("verify_step", oracle.verify(qv, oracle.BF16, kv_v, [NV], scale)),
               ("verify", oracle.verify(qv3, oracle.BF16, kv_v, [NV], scale)))
    for name, (ref_o, ref_l) in checks:
        rows = ref_o.shape[1]
        o = _load(d, f"out_{name}.bin", np.float32, (1, rows, HQ, D)).astype(np.float64)
        l = _load(d, f"lse_{name}.bin", np.float32, (1, rows, HQ)).astype(np.float64)
        err, lerr = np.max(np.abs(o - ref_o)), np.max(np.abs(l - ref_l))
        say(f"  {name}: max|out-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}")
        assert err <= TOL["bf16"] and lerr <= TOL["bf16"], name
    # the ring holds the sinks and the last W positions at their slots, bit for bit
    model = oracle.RingModel(1, S, W)
    model.append(0, N)
    assert np.array_equal(_load(d, "ring_pos.bin", np.int32, (1, S + W)).astype(np.int64),
                          model.tags)
    rk, rv = oracle.ring_expected(model, kv)
    occ = model.occupied_slots(0)
    assert np.array_equal(_load(d, "ring_k.bin", np.uint16, (1, HKV, S + W, D))[0][:, occ],
                          rk[0][:, occ])
    assert np.array_equal(_load(d, "ring_v.bin", np.uint16, (1, HKV, S + W, D))[0][:, occ],
                          rv[0][:, occ])
    assert _load(d, "ring_len.bin", np.int32, (1,))[0] == N
    assert _load(d, "cache_len.bin", np.int32, (1,))[0] == N
    # the verification step stored the candidates after the prefix, bit for bit
    assert np.array_equal(_load(d, "verify_k.bin", np.uint16, (1, HKV, NV_CAP, D))[:, :, :NV], KV_)
    assert np.array_equal(_load(d, "verify_v.bin", np.uint16, (1, HKV, NV_CAP, D))[:, :, :NV], VV_)
    assert _load(d, "verify_len.bin", np.int32, (1,))[0] == NV

    # the speculative iteration on the ring with slack: the allocation-free draft step attended
    # the sinks and the last W of the N + 1 tokens
    kd = _load(d, "k_draft.bin", np.uint16, (1, HKV, D))
    vd = _load(d, "v_draft.bin", np.uint16, (1, HKV, D))
    qd = _load(d, "q_draft.bin", np.uint16, (1, 1, HQ, D))
    K1 = np.concatenate([K, np.ascontiguousarray(kd.transpose(1, 0, 2))[None]], axis=2)
    V1 = np.concatenate([V, np.ascontiguousarray(vd.transpose(1, 0, 2))[None]], axis=2)
    kv1 = oracle.contiguous_kv(K1, V1, oracle.BF16)
    ref_o, ref_l = oracle.draft_windowed(qd, oracle.BF16, kv1, [N + 1], S, W, scale)
    o = _load(d, "out_noalloc.bin", np.float32, (1, 1, HQ, D)).astype(np.float64)
    l = _load(d, "lse_noalloc.bin", np.float32, (1, 1, HQ)).astype(np.float64)
    err, lerr = np.max(np.abs(o - ref_o)), np.max(np.abs(l - ref_l))
    say(f"  allocation-free draft step: max|out-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]
    # greedy accept: exactly the textbook rule on the same logits and drafts
    logits = _load(d, "logits.bin", np.float32, (1, K_ACC + 1, VOCAB))
    drafts = _load(d, "drafts.bin", np.int32, (1, K_ACC))
    choice, n_acc, nxt, n_drop = oracle.greedy_accept(logits, drafts)
    assert np.array_equal(_load(d, "choice.bin", np.int32, (1, K_ACC + 1)), choice)
    assert _load(d, "n_accept.bin", np.int32, (1,))[0] == n_acc[0]
    assert _load(d, "next_token.bin", np.int32, (1,))[0] == nxt[0]
    assert _load(d, "n_drop.bin", np.int32, (1,))[0] == n_drop[0]
    say(f"  greedy accept: {n_acc[0]} of {K_ACC} drafts accepted, {n_drop[0]} rolled back")
    # the rollback by that count: tags, length and the held rows as the host ring model has them
    model2 = oracle.RingModel(1, S, W, SLACK)
    model2.append(0, N + 1)
    model2.rollback(0, int(n_drop[0]))
    assert np.array_equal(_load(d, "ring2_pos.bin", np.int32, (1, S + W + SLACK)).astype(np.int64),
                          model2.tags)
    assert _load(d, "ring2_len.bin", np.int32, (1,))[0] == model2.n[0]
    rk2, rv2 = oracle.ring_expected(model2, kv1)
    occ2 = model2.occupied_slots(0)
    assert np.array_equal(_load(d, "ring2_k.bin", np.uint16, (1, HKV, S + W + SLACK, D))[0][:, occ2],
                          rk2[0][:, occ2])
    assert np.array_equal(_load(d, "ring2_v.bin", np.uint16, (1, HKV, S + W + SLACK, D))[0][:, occ2],
                          rv2[0][:, occ2])
    # MASW-style read: the compact ring's sinks and window plus the NSLOT memory slots
    sk = _load(d, "slots_k.bin", np.uint16, (NSLOT, HKV, D))
    sv = _load(d, "slots_v.bin", np.uint16, (NSLOT, HKV, D))
    ref_o, ref_l = oracle.draft_masw(q, oracle.BF16, kv, [N], S, W,
                                     np.ascontiguousarray(sk.transpose(1, 0, 2))[None],
                                     np.ascontiguousarray(sv.transpose(1, 0, 2))[None], [NSLOT],
                                     scale)
    o = _load(d, "out_masw.bin", np.float32, (1, 1, HQ, D)).astype(np.float64)
    l = _load(d, "lse_masw.bin", np.float32, (1, 1, HQ)).astype(np.float64)
    err, lerr = np.max(np.abs(o - ref_o)), np.max(np.abs(l - ref_l))
    say(f"  masw: max|out-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= TOL["bf16"]
