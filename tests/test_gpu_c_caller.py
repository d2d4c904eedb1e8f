"""A plain C program calls libwmtp.so (tests/c_caller/wmtp_c_caller.c: HIP runtime memory, no
torch, no Python): its ring bytes, position tags, lengths and attention outputs (windowed and
full draft reads, the target's append + verification of 8 candidates and a verification of the
last 3 positions) match the host ring model and the float64 oracle on the same inputs, which the
program writes out."""
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
