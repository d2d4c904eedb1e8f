"""Seeded, counter-based synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module holds no attention arithmetic: it only turns (seed, tensor id, coordinates) into
numbers. Every element is a pure function of its logical coordinates, so any slice of a tensor
(for example the sink and window rows of a million-token prefix) can be produced without
materialising the rest.

Element generator (our own construction from two published pieces):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): ``mix(z)`` is its output finaliser; the stream for a key is
  ``mix(key + (i + 1) * 0x9E3779B97F4A7C15)`` for counter i.
* Box-Muller transform: two 24-bit uniforms u1 in (0,1], u2 in [0,1) from the hash give
  ``sqrt(-2 ln u1) * cos(2 pi u2)`` ~ N(0,1), computed in float64 and rounded once to float32.

bf16 tensors are the float32 draws rounded to nearest-even by torch. The same generator runs on
the CPU or on the GPU (torch int64 arithmetic wraps modulo 2**64 on both); callers hand the same
bytes to both sides, so a last-ulp difference between devices in ``log``/``cos`` never matters.

Tensor ids: Q=0, K=1, V=2, K_new=3, V_new=4, lengths=5 (by convention of the callers).
"""
from __future__ import annotations

import math
from typing import Optional

import torch

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# logical coordinate spans of the counter: b < 2**20, position < 2**22, head < 2**8, dim < 2**10
_POS_BITS, _HEAD_BITS, _DIM_BITS = 22, 8, 10

Q_ID, K_ID, V_ID, KNEW_ID, VNEW_ID, LEN_ID = 0, 1, 2, 3, 4, 5


def _i64(x: int) -> int:
    """Two's-complement int64 with the bits of the unsigned 64-bit value x."""
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output finaliser on int64 bit patterns (wrapping arithmetic)."""
    z = (z ^ _srl(z, 30)) * _i64(_M1)
    z = (z ^ _srl(z, 27)) * _i64(_M2)
    return z ^ _srl(z, 31)


def mix64_int(z: int) -> int:
    """The same finaliser on a Python int (reference for tests and for scalar keys)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    return mix64_int(mix64_int(seed * 0x100 + tensor_id) + _GAMMA)


def hash_counters(seed: int, tensor_id: int, ctr: torch.Tensor) -> torch.Tensor:
    """64-bit hashes (as int64) of counters ``ctr`` in the stream (seed, tensor_id)."""
    key = _i64(stream_key(seed, tensor_id))
    return mix64(key + (ctr + 1) * _i64(_GAMMA))


def normal_from_hash(h: torch.Tensor) -> torch.Tensor:
    """Box-Muller N(0,1) draw (float32) from a 64-bit hash."""
    u1 = (_srl(h, 40).to(torch.float64) + 1.0) * (1.0 / 16777216.0)  # (0, 1]
    u2 = ((h >> 16) & 0xFFFFFF).to(torch.float64) * (1.0 / 16777216.0)  # [0, 1)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return z.to(torch.float32)


def counter(b, pos, head, dim) -> torch.Tensor:
    """Logical counter of element (b, pos, head, dim); arguments broadcast (int64 tensors)."""
    return (((b << _POS_BITS) + pos) << (_HEAD_BITS + _DIM_BITS)) + (head << _DIM_BITS) + dim


def normal_rows(seed: int, tensor_id: int, b: int, positions: torch.Tensor, n_heads: int,
                dim: int, device=None, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """float32 N(0,1) draws for sequence b at the given positions: ``[len(positions)][H][dim]``.
    Generated in chunks so the int64 temporaries stay bounded."""
    device = positions.device if device is None else torch.device(device)
    positions = positions.to(device=device, dtype=torch.int64)
    npos = positions.numel()
    out = torch.empty((npos, n_heads, dim), dtype=torch.float32, device=device)
    if npos == 0:
        return out
    per_row = n_heads * dim
    rows_per_chunk = max(1, chunk_elems // per_row)
    h = torch.arange(n_heads, device=device, dtype=torch.int64).view(1, n_heads, 1)
    i = torch.arange(dim, device=device, dtype=torch.int64).view(1, 1, dim)
    for r0 in range(0, npos, rows_per_chunk):
        p = positions[r0:r0 + rows_per_chunk].view(-1, 1, 1)
        ctr = counter(b, p, h, i)
        out[r0:r0 + rows_per_chunk] = normal_from_hash(hash_counters(seed, tensor_id, ctr))
    return out


def cast(x: torch.Tensor, dtype: torch.dtype, scale: Optional[float] = None) -> torch.Tensor:
    """Optional float32 scaling (one rounding), then conversion (RNE) to the storage dtype."""
    if scale is not None:
        x = x * torch.tensor(scale, dtype=torch.float32, device=x.device)
    return x.to(dtype)


def uniform_int(seed: int, tensor_id: int, index: int, lo: int, hi: int) -> int:
    """Integer in [lo, hi] from the stream (seed, tensor_id) at counter ``index``
    (used for per-sequence lengths). Computed on the host in Python ints."""
    key = stream_key(seed, tensor_id)
    h = mix64_int(key + (index + 1) * _GAMMA)
    return lo + (h % (hi - lo + 1))


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 tensor's bits (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def host_array(t: torch.Tensor):
    """numpy view of a tensor for the oracle: float32 stays float32, bf16 becomes its bits."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()


def sequence_rows(seed: int, tensor_id: int, b: int, p0: int, p1: int, n_heads: int, dim: int,
                  dtype: torch.dtype, device, scale: Optional[float] = None) -> torch.Tensor:
    """Rows of positions [p0, p1) of sequence b, head-major ``[n_heads][p1-p0][dim]`` in the
    storage dtype (the layout of one sequence of a KV cache)."""
    pos = torch.arange(p0, p1, dtype=torch.int64, device=device)
    x = normal_rows(seed, tensor_id, b, pos, n_heads, dim, device)
    return cast(x, dtype, scale).permute(1, 0, 2).contiguous()


def token_rows(seed: int, tensor_id: int, b: int, p0: int, p1: int, n_heads: int, dim: int,
               dtype: torch.dtype, device, scale: Optional[float] = None) -> torch.Tensor:
    """The same rows token-major ``[p1-p0][n_heads][dim]`` (the layout of appended tokens)."""
    pos = torch.arange(p0, p1, dtype=torch.int64, device=device)
    return cast(normal_rows(seed, tensor_id, b, pos, n_heads, dim, device), dtype, scale)


def queries(seed: int, step: int, batch: int, m: int, n_heads: int, dim: int,
            dtype: torch.dtype, device) -> torch.Tensor:
    """Query tensor ``[batch][m][n_heads][dim]`` of draft/verify step ``step``: the m query
    tokens of sequence b are counter positions step*m .. step*m+m-1 of the Q stream."""
    out = torch.empty((batch, m, n_heads, dim), dtype=dtype, device=device)
    for b in range(batch):
        pos = torch.arange(step * m, step * m + m, dtype=torch.int64, device=device)
        out[b] = cast(normal_rows(seed, Q_ID, b, pos, n_heads, dim, device), dtype)
    return out
