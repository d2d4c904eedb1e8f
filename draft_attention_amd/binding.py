"""Thin ctypes binding of libwmtp.so (include/wmtp.h). Argument marshalling only: every step of
the attention and ring paths runs in the HIP kernels behind the C ABI; there is no fallback.

The functions carry the C names. They accept torch tensors (device memory owned by the caller)
and pass their data pointers, plus the current torch stream unless a stream is given. They return
the wmtp status code; with ``check=True`` (the default) a nonzero status raises :class:`WmtpError`.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# WMTP_LIB names another build of the same sources to load (e.g. one with host-side sanitizers)
LIB_PATH = os.environ.get("WMTP_LIB") or os.path.join(_HERE, "libwmtp.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "wmtp.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(_HERE), "include", "wmtp_probe.h")]

WMTP_OK = 0
WMTP_ERR_INVALID_ARG = 1
WMTP_ERR_UNSUPPORTED = 2
WMTP_ERR_CAPACITY = 3
WMTP_ERR_WORKSPACE = 4
WMTP_ERR_HIP = 5
WMTP_F32 = 0
WMTP_BF16 = 1


class WmtpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class wmtp_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("sink", ctypes.c_int32),
                ("window", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libwmtp.so. Raises if it has not been built: there is no other implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_attention_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        kvp = ctypes.POINTER(wmtp_kv)
        L.wmtp_ring_append.argtypes = [kvp, vp, vp, i32, vp]
        L.wmtp_draft_attn_windowed.argtypes = [kvp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.wmtp_draft_attn_full.argtypes = [kvp, vp, i32, f32, i32, vp, vp, vp, sz, vp]
        L.wmtp_verify_attn.argtypes = [kvp, vp, i32, i32, f32, i32, vp, vp, vp, sz, vp]
        L.wmtp_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.wmtp_attn_workspace_bytes.restype = sz
        L.wmtp_status_string.argtypes = [ctypes.c_int]
        L.wmtp_status_string.restype = ctypes.c_char_p
        L.wmtp_ring_rollback.argtypes = [kvp, vp, vp]
        L.wmtp_draft_step_windowed.argtypes = [kvp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.wmtp_draft_step_full.argtypes = [kvp, vp, vp, vp, i32, f32, i32, vp, vp, vp, sz, vp]
        L.wmtp_verify_step.argtypes = [kvp, vp, vp, vp, i32, i32, f32, i32, vp, vp, vp, sz, vp]
        L.wmtp_draft_step_windowed_noalloc.argtypes = [kvp, vp, vp, vp, i32, f32, vp, vp, vp]
        L.wmtp_draft_attn_masw.argtypes = [kvp, kvp, vp, i32, f32, i32, vp, vp, vp, sz, vp]
        L.wmtp_masw_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.wmtp_masw_workspace_bytes.restype = sz
        L.wmtp_greedy_accept.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.wmtp_accept_workspace_bytes.argtypes = [i32, i32, i32]
        L.wmtp_accept_workspace_bytes.restype = sz
        L.wmtp_probe_read.argtypes = [vp, sz, vp, vp]
        L.wmtp_llc_flush.argtypes = [vp, sz, ctypes.c_uint8, vp]
        L.wmtp_probe_handoff.argtypes = [vp, sz, i32, vp, sz, vp, vp]
        for name in ("wmtp_ring_append", "wmtp_draft_attn_windowed", "wmtp_draft_attn_full",
                     "wmtp_verify_attn", "wmtp_ring_rollback", "wmtp_greedy_accept",
                     "wmtp_draft_attn_masw", "wmtp_draft_step_windowed", "wmtp_draft_step_full",
                     "wmtp_verify_step", "wmtp_draft_step_windowed_noalloc",
                     "wmtp_probe_read", "wmtp_probe_handoff", "wmtp_llc_flush"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/wmtp.h and include/wmtp_probe.h declare."""
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(wmtp_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().wmtp_status_string(int(status)).decode()


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None stays NULL; ints pass through as raw addresses)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("wmtp: every buffer must be device memory (got a host tensor)")
    if not t.is_contiguous():
        raise ValueError("wmtp: buffers must be dense (contiguous) tensors")
    return t.data_ptr()


_current_stream = None


def _stream(stream) -> Optional[int]:
    """The hipStream_t to enqueue on: the given stream, else torch's current stream of the current
    device (looked up through torch's raw-handle accessor when it has one: constructing a
    torch.cuda.Stream object per call costs a few microseconds of host time)."""
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    global _current_stream
    if _current_stream is None:
        import torch

        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        if raw is not None and dev is not None:
            _current_stream = lambda: raw(dev())
        else:
            _current_stream = lambda: torch.cuda.current_stream().cuda_stream
    return _current_stream()


def _done(status: int, what: str, check: bool) -> int:
    if check and status != WMTP_OK:
        raise WmtpError(status, what)
    return status


@dataclass(eq=False)
class KVCache:
    """Device tensors of one cache plus its geometry; ``desc()`` gives the C descriptor.

    The descriptor is validated and built on first use and kept until a field is reassigned, so
    a cache tensor must not be resized or re-pointed in place (``resize_``, ``set_``) once the
    cache has been used; assign a new tensor to the field instead."""

    k: object
    v: object
    pos: object
    seq_len: object
    batch: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    sink: int
    window: int
    dtype: int

    @classmethod
    def allocate(cls, batch, n_kv_heads, head_dim, capacity, sink, window, torch_dtype,
                 device="cuda", with_pos=True):
        """Zeroed cache tensors (torch owns the memory). Ring: window >= 1 and
        capacity >= sink + window; contiguous: window = 0 and sink = capacity."""
        import torch

        shape = (batch, n_kv_heads, capacity, head_dim)
        k = torch.zeros(shape, dtype=torch_dtype, device=device)
        v = torch.zeros(shape, dtype=torch_dtype, device=device)
        pos = (torch.full((batch, capacity), -1, dtype=torch.int32, device=device)
               if with_pos else None)
        seq_len = torch.zeros(batch, dtype=torch.int32, device=device)
        return cls(k, v, pos, seq_len, batch, n_kv_heads, head_dim, capacity, sink, window,
                   dtype_code(torch_dtype))

    @classmethod
    def ring(cls, batch, n_kv_heads, head_dim, sink, window, torch_dtype, device="cuda",
             with_pos=True, slack=0):
        """A ring of sink + window + slack slots (slack > 0 allows rolling back that many of the
        newest tokens)."""
        return cls.allocate(batch, n_kv_heads, head_dim, sink + window + slack, sink, window,
                            torch_dtype, device, with_pos)

    @classmethod
    def contiguous(cls, batch, n_kv_heads, head_dim, capacity, torch_dtype, device="cuda",
                   with_pos=False):
        return cls.allocate(batch, n_kv_heads, head_dim, capacity, capacity, 0, torch_dtype,
                            device, with_pos)

    def __setattr__(self, name, value):
        object.__setattr__(self, name, value)
        if name != "_c":
            object.__setattr__(self, "_c", None)  # geometry or a tensor changed: rebuild

    def desc(self) -> wmtp_kv:
        c = self.__dict__.get("_c")
        if c is None:
            # the cache tensors must be device memory, dense, and as large as the geometry says
            # (the kernels index them by it)
            eb = 2 if self.dtype == WMTP_BF16 else 4
            rows = self.batch * self.n_kv_heads * self.capacity * self.head_dim
            _numel_ok(self.k, rows, eb, "cache.k")
            _numel_ok(self.v, rows, eb, "cache.v")
            _numel_ok(self.pos, self.batch * self.capacity, 4, "cache.pos")
            _numel_ok(self.seq_len, self.batch, 4, "cache.seq_len")
            c = wmtp_kv(_ptr(self.k), _ptr(self.v), _ptr(self.pos), _ptr(self.seq_len),
                        self.batch, self.n_kv_heads, self.head_dim, self.capacity, self.sink,
                        self.window, self.dtype)
            object.__setattr__(self, "_c", c)
        return c


def dtype_code(torch_dtype) -> int:
    import torch

    if torch_dtype == torch.float32:
        return WMTP_F32
    if torch_dtype == torch.bfloat16:
        return WMTP_BF16
    raise ValueError(f"unsupported dtype {torch_dtype}")


def _desc(cache):
    return cache.desc() if isinstance(cache, KVCache) else cache


def _numel_ok(t, count: int, elem_bytes: int, name: str) -> None:
    """A tensor handed to the library must hold at least the elements the call reads or writes
    (the device cannot check this)."""
    if t is None or isinstance(t, int):
        return
    if t.element_size() != elem_bytes:
        raise ValueError(f"wmtp: {name} has {t.element_size()}-byte elements, expected {elem_bytes}")
    if t.numel() < count:
        raise ValueError(f"wmtp: {name} holds {t.numel()} elements, the call needs {count}")


def _check_attn(d: wmtp_kv, q, m: int, n_q_heads: int, out, lse) -> None:
    eb = 2 if d.dtype == WMTP_BF16 else 4
    rows = d.batch * m * n_q_heads
    _numel_ok(q, rows * d.head_dim, eb, "q")
    _numel_ok(out, rows * d.head_dim, 4, "out")
    _numel_ok(lse, rows, 4, "lse")


def _check_append(d: wmtp_kv, k_new, v_new, n_new: int) -> None:
    eb = 2 if d.dtype == WMTP_BF16 else 4
    count = d.batch * max(n_new, 0) * d.n_kv_heads * d.head_dim
    _numel_ok(k_new, count, eb, "k_new")
    _numel_ok(v_new, count, eb, "v_new")


# ------------------------------------------------------------------------------------------
# the C ABI, one function each
# ------------------------------------------------------------------------------------------
def wmtp_ring_append(cache, k_new, v_new, n_new: int, stream=None, check=True) -> int:
    d = _desc(cache)
    _check_append(d, k_new, v_new, n_new)
    st = lib().wmtp_ring_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), int(n_new),
                                _stream(stream))
    return _done(st, "wmtp_ring_append", check)


def wmtp_draft_attn_windowed(ring, q, n_q_heads: int, sm_scale: float, out, lse, ws,
                             ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    d = _desc(ring)
    _check_attn(d, q, 1, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_draft_attn_windowed(ctypes.byref(d), _ptr(q), int(n_q_heads), float(sm_scale),
                                        _ptr(out), _ptr(lse), _ptr(ws), int(nbytes),
                                        _stream(stream))
    return _done(st, "wmtp_draft_attn_windowed", check)


def wmtp_draft_attn_full(cache, q, n_q_heads: int, sm_scale: float, max_seq_len: int, out, lse,
                         ws, ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    d = _desc(cache)
    _check_attn(d, q, 1, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_draft_attn_full(ctypes.byref(d), _ptr(q), int(n_q_heads), float(sm_scale),
                                    int(max_seq_len), _ptr(out), _ptr(lse), _ptr(ws), int(nbytes),
                                    _stream(stream))
    return _done(st, "wmtp_draft_attn_full", check)


def wmtp_verify_attn(cache, q, m: int, n_q_heads: int, sm_scale: float, max_seq_len: int, out,
                     lse, ws, ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    d = _desc(cache)
    _check_attn(d, q, m, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_verify_attn(ctypes.byref(d), _ptr(q), int(m), int(n_q_heads),
                                float(sm_scale), int(max_seq_len), _ptr(out), _ptr(lse),
                                _ptr(ws), int(nbytes), _stream(stream))
    return _done(st, "wmtp_verify_attn", check)


WMTP_PROBE_BLOCKS = 512  # include/wmtp_probe.h


def wmtp_probe_read(buf, out, nbytes: Optional[int] = None, stream=None, check=True) -> int:
    """Stream `nbytes` (default: all) of `buf` once; out gets WMTP_PROBE_BLOCKS uint32 XORs."""
    _numel_ok(out, WMTP_PROBE_BLOCKS, 4, "out")
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if not isinstance(buf, int) and n > buf.numel() * buf.element_size():
        raise ValueError("wmtp: nbytes exceeds the buffer")
    st = lib().wmtp_probe_read(_ptr(buf), int(n), _ptr(out), _stream(stream))
    return _done(st, "wmtp_probe_read", check)


WMTP_PROBE_HANDOFF_BLOCKS = 256  # include/wmtp_probe.h


def wmtp_probe_handoff(buf, n_groups: int, parts, part_bytes: int, out, nbytes: Optional[int] = None,
                       stream=None, check=True) -> int:
    """Two launches without arithmetic: n_groups workgroups read `nbytes` (default: all) of `buf`,
    each writing `part_bytes` of partials into `parts`; then WMTP_PROBE_HANDOFF_BLOCKS workgroups
    read the partials back, out getting one uint32 XOR each."""
    _numel_ok(out, WMTP_PROBE_HANDOFF_BLOCKS, 4, "out")
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if not isinstance(buf, int) and n > buf.numel() * buf.element_size():
        raise ValueError("wmtp: nbytes exceeds the buffer")
    if not isinstance(parts, int) and n_groups * part_bytes > parts.numel() * parts.element_size():
        raise ValueError("wmtp: parts holds fewer than n_groups * part_bytes bytes")
    st = lib().wmtp_probe_handoff(_ptr(buf), int(n), int(n_groups), _ptr(parts), int(part_bytes),
                                  _ptr(out), _stream(stream))
    return _done(st, "wmtp_probe_handoff", check)


def wmtp_llc_flush(buf, value: int = 0, stream=None, check=True) -> int:
    """Overwrite all of `buf` with the byte `value` (evicts earlier calls' lines from the caches)."""
    n = buf.numel() * buf.element_size()
    st = lib().wmtp_llc_flush(_ptr(buf), int(n), int(value) & 0xFF, _stream(stream))
    return _done(st, "wmtp_llc_flush", check)


def wmtp_draft_step_windowed(ring, k_new, v_new, q, n_q_heads: int, sm_scale: float, out, lse, ws,
                             ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    """Append one token per sequence, then the windowed draft attention (one call)."""
    d = _desc(ring)
    _check_append(d, k_new, v_new, 1)
    _check_attn(d, q, 1, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_draft_step_windowed(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q),
                                        int(n_q_heads), float(sm_scale), _ptr(out), _ptr(lse),
                                        _ptr(ws), int(nbytes), _stream(stream))
    return _done(st, "wmtp_draft_step_windowed", check)


def wmtp_draft_step_windowed_noalloc(ring, k_new, v_new, q, n_q_heads: int, sm_scale: float, out,
                                     lse, stream=None, check=True) -> int:
    """wmtp_draft_step_windowed with the partials in the library's static device scratch (no
    workspace; allocates nothing)."""
    d = _desc(ring)
    _check_append(d, k_new, v_new, 1)
    _check_attn(d, q, 1, n_q_heads, out, lse)
    st = lib().wmtp_draft_step_windowed_noalloc(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q),
                                                int(n_q_heads), float(sm_scale), _ptr(out),
                                                _ptr(lse), _stream(stream))
    return _done(st, "wmtp_draft_step_windowed_noalloc", check)


def wmtp_draft_step_full(cache, k_new, v_new, q, n_q_heads: int, sm_scale: float,
                         max_seq_len: int, out, lse, ws, ws_bytes: Optional[int] = None,
                         stream=None, check=True) -> int:
    """Append one token per sequence, then the full-context draft attention (one call)."""
    d = _desc(cache)
    _check_append(d, k_new, v_new, 1)
    _check_attn(d, q, 1, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_draft_step_full(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q),
                                    int(n_q_heads), float(sm_scale), int(max_seq_len), _ptr(out),
                                    _ptr(lse), _ptr(ws), int(nbytes), _stream(stream))
    return _done(st, "wmtp_draft_step_full", check)


def wmtp_verify_step(cache, k_new, v_new, q, m: int, n_q_heads: int, sm_scale: float,
                     max_seq_len: int, out, lse, ws, ws_bytes: Optional[int] = None, stream=None,
                     check=True) -> int:
    """Append the m candidates, then verify them (one call)."""
    d = _desc(cache)
    _check_append(d, k_new, v_new, m)
    _check_attn(d, q, m, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_verify_step(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(q), int(m),
                                int(n_q_heads), float(sm_scale), int(max_seq_len), _ptr(out),
                                _ptr(lse), _ptr(ws), int(nbytes), _stream(stream))
    return _done(st, "wmtp_verify_step", check)


def wmtp_draft_attn_masw(ring, slots, q, n_q_heads: int, sm_scale: float, max_slots: int, out,
                         lse, ws, ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    """MASW draft step: ring sinks + last W positions, plus memory slots 0..slots.seq_len[b]-1."""
    r, sl = _desc(ring), _desc(slots)
    _check_attn(r, q, 1, n_q_heads, out, lse)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_draft_attn_masw(ctypes.byref(r), ctypes.byref(sl), _ptr(q), int(n_q_heads),
                                    float(sm_scale), int(max_slots), _ptr(out), _ptr(lse),
                                    _ptr(ws), int(nbytes), _stream(stream))
    return _done(st, "wmtp_draft_attn_masw", check)


def wmtp_masw_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, ring_capacity,
                              max_slots) -> int:
    return int(lib().wmtp_masw_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                               ring_capacity, max_slots))


def masw_workspace(batch, n_q_heads, n_kv_heads, head_dim, ring_capacity, max_slots,
                   device="cuda"):
    import torch

    n = wmtp_masw_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, ring_capacity, max_slots)
    if n == 0:
        raise ValueError("wmtp_draft_attn_masw does not accept these sizes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def wmtp_ring_rollback(cache, n_drop, stream=None, check=True) -> int:
    """Discard the newest n_drop[b] tokens of every sequence (device int32 [batch])."""
    d = _desc(cache)
    _numel_ok(n_drop, d.batch, 4, "n_drop")
    st = lib().wmtp_ring_rollback(ctypes.byref(d), _ptr(n_drop), _stream(stream))
    return _done(st, "wmtp_ring_rollback", check)


def wmtp_accept_workspace_bytes(batch: int, k: int, vocab: int) -> int:
    return int(lib().wmtp_accept_workspace_bytes(batch, k, vocab))


def wmtp_greedy_accept(logits, k: int, draft_tokens, choice, n_accept, next_token, n_drop, ws,
                       ws_bytes: Optional[int] = None, stream=None, check=True) -> int:
    """Greedy verification: logits [B][k+1][V] (float32 or bfloat16), draft_tokens [B][k] int32;
    writes choice [B][k+1], n_accept, next_token and n_drop [B] (int32)."""
    B, k1, V = (int(x) for x in logits.shape)
    if k1 != k + 1:
        raise ValueError("logits must hold k + 1 rows per sequence")
    code = dtype_code(logits.dtype)
    _numel_ok(logits, B * k1 * V, 2 if code == WMTP_BF16 else 4, "logits")
    if k > 0:
        _numel_ok(draft_tokens, B * k, 4, "draft_tokens")
    _numel_ok(choice, B * k1, 4, "choice")
    for t, name in ((n_accept, "n_accept"), (next_token, "next_token"), (n_drop, "n_drop")):
        _numel_ok(t, B, 4, name)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    st = lib().wmtp_greedy_accept(_ptr(logits), code, B, int(k), V,
                                  _ptr(draft_tokens) if k > 0 else None, _ptr(choice),
                                  _ptr(n_accept), _ptr(next_token), _ptr(n_drop), _ptr(ws),
                                  int(nbytes), _stream(stream))
    return _done(st, "wmtp_greedy_accept", check)


def accept_workspace(batch: int, k: int, vocab: int, device="cuda"):
    """A 256-byte-aligned device byte tensor large enough for wmtp_greedy_accept."""
    import torch

    n = wmtp_accept_workspace_bytes(batch, k, vocab)
    if n == 0:
        raise ValueError("wmtp_greedy_accept does not accept these sizes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def wmtp_attn_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, m: int,
                              max_seq_len: int) -> int:
    return int(lib().wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, m,
                                               max_seq_len))


def wmtp_status_string(status: int) -> str:
    return status_string(status)


def workspace(batch, n_q_heads, n_kv_heads, head_dim, m, max_seq_len, device="cuda"):
    """A device byte tensor large enough for an attention call with these sizes."""
    import torch

    n = wmtp_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, m, max_seq_len)
    if n == 0:
        raise ValueError("no attention call accepts these sizes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]
