"""Helpers for the GPU tests: build caches through the C ABI from seeded synthetic sequences and
compare the HIP results with the float64 oracle on the same bytes."""
from __future__ import annotations

import math
import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
from draft_attention_amd import binding as W
from draft_attention_amd import synth

# tolerances on max |gpu - oracle| (float32 inputs; bf16 inputs with float32 accumulation)
TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda"


def tdtype(name: str):
    return torch.float32 if name == "f32" else torch.bfloat16


def ocode(name: str) -> int:
    return oracle.F32 if name == "f32" else oracle.BF16


def say(msg: str) -> None:
    """Name the case before GPU work, so a failing run leaves a trace."""
    print(msg, file=sys.stderr, flush=True)


def logical_kv(seed, batch, n_kv_heads, head_dim, length, dt, k_scale=None, device=DEV):
    """Logical K/V ``[B][Hkv][length][d]`` of positions 0..length-1 on the device."""
    K = torch.stack([synth.sequence_rows(seed, synth.K_ID, b, 0, length, n_kv_heads, head_dim,
                                         dt, device, k_scale) for b in range(batch)])
    V = torch.stack([synth.sequence_rows(seed, synth.V_ID, b, 0, length, n_kv_heads, head_dim,
                                         dt, device) for b in range(batch)])
    return K, V


def oracle_kv(K: torch.Tensor, V: torch.Tensor, dtname: str) -> oracle.LogicalKV:
    return oracle.contiguous_kv(synth.host_array(K), synth.host_array(V), ocode(dtname))


def select(cache: W.KVCache, b: int) -> W.KVCache:
    """Batch-1 view of sequence b (pointers offset into the same tensors)."""
    return W.KVCache(cache.k[b:b + 1], cache.v[b:b + 1],
                     None if cache.pos is None else cache.pos[b:b + 1], cache.seq_len[b:b + 1],
                     1, cache.n_kv_heads, cache.head_dim, cache.capacity, cache.sink,
                     cache.window, cache.dtype)


def tokens(K: torch.Tensor, b: int, p0: int, p1: int) -> torch.Tensor:
    """Token-major rows ``[p1-p0][Hkv][d]`` of positions [p0, p1) of sequence b."""
    return K[b, :, p0:p1].permute(1, 0, 2).contiguous()


def append_each(cache: W.KVCache, K, V, lens: Sequence[int], counts: Sequence[int]):
    """Append counts[b] tokens to sequence b (its next positions lens[b]..), one call per
    sequence through a batch-1 descriptor."""
    for b, t in enumerate(counts):
        if t == 0:
            continue
        sub = select(cache, b)
        kn = tokens(K, b, lens[b], lens[b] + t)[None]
        vn = tokens(V, b, lens[b], lens[b] + t)[None]
        W.wmtp_ring_append(sub, kn, vn, t)


def append_all(cache: W.KVCache, K, V, lens: Sequence[int], t: int):
    """Append t tokens to every sequence in one call (sequence b gets positions lens[b]..)."""
    kn = torch.stack([tokens(K, b, lens[b], lens[b] + t) for b in range(cache.batch)])
    vn = torch.stack([tokens(V, b, lens[b], lens[b] + t) for b in range(cache.batch)])
    W.wmtp_ring_append(cache, kn, vn, t)


def run_windowed(ring: W.KVCache, q: torch.Tensor, n_q_heads: int, scale: float):
    B, d = ring.batch, ring.head_dim
    out = torch.full((B, 1, n_q_heads, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, 1, n_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = W.workspace(B, n_q_heads, ring.n_kv_heads, d, 1, ring.capacity)
    W.wmtp_draft_attn_windowed(ring, q, n_q_heads, scale, out, lse, ws)
    return out, lse


def run_full(cache: W.KVCache, q: torch.Tensor, n_q_heads: int, scale: float, max_seq_len: int):
    B, d = cache.batch, cache.head_dim
    out = torch.full((B, 1, n_q_heads, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, 1, n_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = W.workspace(B, n_q_heads, cache.n_kv_heads, d, 1, max_seq_len)
    W.wmtp_draft_attn_full(cache, q, n_q_heads, scale, max_seq_len, out, lse, ws)
    return out, lse


def run_verify(cache: W.KVCache, q: torch.Tensor, n_q_heads: int, scale: float,
               max_seq_len: int):
    B, m, d = cache.batch, q.shape[1], cache.head_dim
    out = torch.full((B, m, n_q_heads, d), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, m, n_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    ws = W.workspace(B, n_q_heads, cache.n_kv_heads, d, m, max_seq_len)
    W.wmtp_verify_attn(cache, q, m, n_q_heads, scale, max_seq_len, out, lse, ws)
    return out, lse


def compare(out: torch.Tensor, lse: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray,
            dtname: str, what: str):
    """Assert max |out - ref| <= tolerance; lse with the same bound; report the errors."""
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness differs"
    lerr = float(np.max(np.abs(l[fin] - ref_lse[fin]))) if fin.any() else 0.0
    tol = TOL[dtname]
    say(f"  {what}: max|out-ref| = {err:.3e}  max|lse-ref| = {lerr:.3e}  (tol {tol:g})")
    assert err <= tol, f"{what}: output error {err} > {tol}"
    assert lerr <= tol, f"{what}: lse error {lerr} > {tol}"
    return err, lerr
