"""The C ABI on the host (no GPU): libwmtp.so loads, exports every function include/wmtp.h
declares, and every invalid argument is refused with its status before anything is launched."""
import ctypes
import math
import os

import pytest

from draft_attention_amd import binding as W

FAKE = 0x10000  # an aligned, non-null address that is never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(W.LIB_PATH):
        from draft_attention_amd import build

        build.build()
    return W.lib()


def _kv(**kw):
    base = dict(k=FAKE, v=FAKE, pos=None, seq_len=FAKE, batch=2, n_kv_heads=2, head_dim=128,
                capacity=20, sink=4, window=16, dtype=W.WMTP_BF16)
    base.update(kw)
    return W.wmtp_kv(**base)


def test_exports_every_declared_function(lib):
    names = W.header_functions()
    assert set(names) == {"wmtp_ring_append", "wmtp_draft_attn_windowed", "wmtp_draft_attn_full",
                          "wmtp_verify_attn", "wmtp_attn_workspace_bytes", "wmtp_status_string",
                          "wmtp_probe_read", "wmtp_probe_handoff", "wmtp_llc_flush",
                          "wmtp_ring_rollback",
                          "wmtp_greedy_accept", "wmtp_accept_workspace_bytes",
                          "wmtp_draft_attn_masw", "wmtp_masw_workspace_bytes",
                          "wmtp_draft_step_windowed", "wmtp_draft_step_full", "wmtp_verify_step",
                          "wmtp_draft_step_windowed_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in range(6):
        assert W.status_string(st).startswith("WMTP_")
    assert "unknown" in W.status_string(99)


def _append(desc, k_new=FAKE, v_new=FAKE, n_new=1):
    return W.lib().wmtp_ring_append(ctypes.byref(desc) if desc is not None else None, k_new,
                                    v_new, n_new, None)


def _windowed(desc, q=FAKE, hq=8, scale=0.1, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return W.lib().wmtp_draft_attn_windowed(ctypes.byref(desc), q, hq, scale, out, None, ws,
                                            ws_bytes, None)


def _full(desc, bound=10, hq=8, ws_bytes=1 << 30, ws=FAKE):
    return W.lib().wmtp_draft_attn_full(ctypes.byref(desc), FAKE, hq, 0.1, bound, FAKE, None, ws,
                                        ws_bytes, None)


def _verify(desc, m=4, bound=10, hq=8, ws_bytes=1 << 30):
    return W.lib().wmtp_verify_attn(ctypes.byref(desc), FAKE, m, hq, 0.1, bound, FAKE, None, FAKE,
                                    ws_bytes, None)


CONTIG = dict(capacity=64, sink=64, window=0)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), W.WMTP_ERR_UNSUPPORTED),
    (dict(head_dim=96), W.WMTP_ERR_UNSUPPORTED),
    (dict(k=None), W.WMTP_ERR_INVALID_ARG),
    (dict(v=None), W.WMTP_ERR_INVALID_ARG),
    (dict(seq_len=None), W.WMTP_ERR_INVALID_ARG),
    (dict(batch=0), W.WMTP_ERR_INVALID_ARG),
    (dict(n_kv_heads=0), W.WMTP_ERR_INVALID_ARG),
    (dict(capacity=19), W.WMTP_ERR_INVALID_ARG),          # ring: capacity < sink + window
    (dict(sink=-1, capacity=15), W.WMTP_ERR_INVALID_ARG),
    (dict(capacity=64, sink=60, window=0), W.WMTP_ERR_INVALID_ARG),  # contiguous: sink != cap
    (dict(k=FAKE + 8), W.WMTP_ERR_INVALID_ARG),           # misaligned
    (dict(pos=FAKE + 2), W.WMTP_ERR_INVALID_ARG),
])
def test_descriptor_validation(lib, kw, status):
    d = _kv(**kw)
    assert _append(d) == status
    assert _windowed(d) == status


def test_append_validation(lib):
    assert lib.wmtp_ring_append(None, FAKE, FAKE, 1, None) == W.WMTP_ERR_INVALID_ARG
    assert _append(_kv(), n_new=-1) == W.WMTP_ERR_INVALID_ARG
    assert _append(_kv(), n_new=0) == W.WMTP_OK  # no-op, nothing launched
    assert _append(_kv(), k_new=None) == W.WMTP_ERR_INVALID_ARG
    assert _append(_kv(), v_new=FAKE + 4) == W.WMTP_ERR_INVALID_ARG
    assert _append(_kv(**CONTIG), n_new=65) == W.WMTP_ERR_CAPACITY


def test_windowed_validation(lib):
    need = W.wmtp_attn_workspace_bytes(2, 8, 2, 128, 1, 20)
    assert need > 0
    assert _windowed(_kv(**CONTIG)) == W.WMTP_ERR_INVALID_ARG       # not a ring
    assert _windowed(_kv(), hq=7) == W.WMTP_ERR_INVALID_ARG          # Hq % Hkv != 0
    assert _windowed(_kv(), hq=1) == W.WMTP_ERR_INVALID_ARG          # Hq < Hkv
    assert _windowed(_kv(), q=None) == W.WMTP_ERR_INVALID_ARG
    assert _windowed(_kv(), out=None) == W.WMTP_ERR_INVALID_ARG
    assert _windowed(_kv(), out=FAKE + 4) == W.WMTP_ERR_INVALID_ARG
    assert _windowed(_kv(), scale=math.nan) == W.WMTP_ERR_INVALID_ARG
    assert _windowed(_kv(), ws=None) == W.WMTP_ERR_WORKSPACE
    assert _windowed(_kv(), ws=FAKE + 16) == W.WMTP_ERR_WORKSPACE    # not 256-byte aligned
    assert _windowed(_kv(), ws_bytes=need - 1) == W.WMTP_ERR_WORKSPACE


def test_full_and_verify_validation(lib):
    c = _kv(**CONTIG)
    assert _full(_kv()) == W.WMTP_ERR_INVALID_ARG                    # a ring is not a full cache
    assert _full(c, bound=0) == W.WMTP_ERR_INVALID_ARG
    assert _full(c, bound=65) == W.WMTP_ERR_INVALID_ARG              # beyond capacity
    assert _full(c, ws_bytes=16) == W.WMTP_ERR_WORKSPACE
    assert _verify(c, m=0) == W.WMTP_ERR_INVALID_ARG
    assert _verify(c, m=17) == W.WMTP_ERR_INVALID_ARG
    assert _verify(_kv()) == W.WMTP_ERR_INVALID_ARG
    assert _verify(c, ws_bytes=16) == W.WMTP_ERR_WORKSPACE


def test_workspace_bytes(lib):
    f = W.wmtp_attn_workspace_bytes
    assert f(1, 8, 2, 96, 1, 100) == 0          # unsupported head_dim
    assert f(1, 7, 2, 128, 1, 100) == 0         # Hq % Hkv
    assert f(1, 8, 2, 128, 0, 100) == 0         # m < 1
    assert f(1, 8, 2, 128, 17, 100) == 0        # m > 16
    assert f(1, 8, 2, 128, 1, 0) == 0
    small, big = f(1, 32, 2, 256, 1, 4100), f(1, 32, 2, 256, 1, 1048581)
    assert 0 < small <= big
    # the split-K partials stay a small fraction of the K/V bytes a full 1M-token read streams
    kv_bytes = 2 * 2 * 1048581 * 256 * 2
    assert big < 0.05 * kv_bytes


def test_probe_arguments_rejected_before_launch(lib):
    out = FAKE
    assert lib.wmtp_probe_read(None, 1024, out, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_probe_read(FAKE, 0, out, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_probe_read(FAKE, 1000, out, None) == W.WMTP_ERR_INVALID_ARG  # not 16-byte sized
    assert lib.wmtp_probe_read(FAKE + 8, 1024, out, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_probe_read(FAKE, 1024, None, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_llc_flush(None, 1024, 0, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_llc_flush(FAKE, 24, 0, None) == W.WMTP_ERR_INVALID_ARG
    assert lib.wmtp_llc_flush(FAKE + 4, 1024, 0, None) == W.WMTP_ERR_INVALID_ARG
    h = lib.wmtp_probe_handoff
    assert h(None, 1024, 4, FAKE, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1000, 4, FAKE, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 0, FAKE, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 65536, FAKE, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 2, FAKE, 8, out, None) == W.WMTP_ERR_INVALID_ARG  # product 16, part not
    assert h(FAKE, 1024, 4, FAKE, 0, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 4, FAKE + 8, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 4, None, 256, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 2, FAKE, 1 << 40, out, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 4, FAKE, 256, None, None) == W.WMTP_ERR_INVALID_ARG
    assert h(FAKE, 1024, 4, FAKE, 256, FAKE + 2, None) == W.WMTP_ERR_INVALID_ARG


def test_ring_with_slack_is_a_valid_descriptor_and_short_capacity_is_not(lib):
    # capacity below sink + window is rejected before anything runs (a NULL k_new fails later)
    assert _append(_kv(capacity=19)) == W.WMTP_ERR_INVALID_ARG
    assert _append(_kv(capacity=24), k_new=None) == W.WMTP_ERR_INVALID_ARG  # slack ring accepted
    assert _windowed(_kv(capacity=24), ws_bytes=0) == W.WMTP_ERR_WORKSPACE


def test_rollback_arguments_rejected_before_launch(lib):
    L = W.lib()
    assert L.wmtp_ring_rollback(None, FAKE, None) == W.WMTP_ERR_INVALID_ARG
    assert L.wmtp_ring_rollback(ctypes.byref(_kv()), None, None) == W.WMTP_ERR_INVALID_ARG
    assert L.wmtp_ring_rollback(ctypes.byref(_kv()), FAKE + 2, None) == W.WMTP_ERR_INVALID_ARG
    assert L.wmtp_ring_rollback(ctypes.byref(_kv(head_dim=96)), FAKE, None) == W.WMTP_ERR_UNSUPPORTED
    # a ring with slack reads its exact rollback depth from the position tags: pos is required
    assert L.wmtp_ring_rollback(ctypes.byref(_kv(capacity=24)), FAKE, None) == W.WMTP_ERR_INVALID_ARG


def test_accept_arguments_rejected_before_launch(lib):
    L = W.lib()
    ws_need = L.wmtp_accept_workspace_bytes(2, 3, 1000)
    assert ws_need > 0
    assert L.wmtp_accept_workspace_bytes(0, 3, 1000) == 0
    assert L.wmtp_accept_workspace_bytes(2, 64, 1000) == 0

    def call(logits=FAKE, dtype=W.WMTP_BF16, batch=2, k=3, vocab=1000, draft=FAKE, out=FAKE,
             ws=FAKE, ws_bytes=1 << 20):
        return L.wmtp_greedy_accept(logits, dtype, batch, k, vocab, draft, out, out, out, out, ws,
                                    ws_bytes, None)

    assert call(dtype=7) == W.WMTP_ERR_UNSUPPORTED
    assert call(logits=None) == W.WMTP_ERR_INVALID_ARG
    assert call(logits=FAKE + 1) == W.WMTP_ERR_INVALID_ARG
    assert call(dtype=W.WMTP_F32, logits=FAKE + 2) == W.WMTP_ERR_INVALID_ARG
    assert call(draft=None) == W.WMTP_ERR_INVALID_ARG
    assert call(k=-1) == W.WMTP_ERR_INVALID_ARG
    assert call(k=64) == W.WMTP_ERR_INVALID_ARG
    assert call(vocab=0) == W.WMTP_ERR_INVALID_ARG
    assert call(out=None) == W.WMTP_ERR_INVALID_ARG
    assert call(ws=None) == W.WMTP_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == W.WMTP_ERR_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == W.WMTP_ERR_WORKSPACE


def test_masw_arguments_rejected_before_launch(lib):
    L = W.lib()
    ring = _kv()
    slots = _kv(**CONTIG)
    need = L.wmtp_masw_workspace_bytes(2, 8, 2, 128, 20, 64)
    assert need > 0

    def call(r=ring, sl=slots, q=FAKE, hq=8, max_slots=64, ws=FAKE, ws_bytes=1 << 30):
        return L.wmtp_draft_attn_masw(ctypes.byref(r), ctypes.byref(sl), q, hq, 0.1, max_slots,
                                      FAKE, None, ws, ws_bytes, None)

    assert call(r=_kv(**CONTIG)) == W.WMTP_ERR_INVALID_ARG       # first cache must be a ring
    assert call(sl=_kv()) == W.WMTP_ERR_INVALID_ARG               # slots must be contiguous
    assert call(sl=_kv(**CONTIG, head_dim=64)) == W.WMTP_ERR_INVALID_ARG
    assert call(sl=_kv(**CONTIG, dtype=W.WMTP_F32)) == W.WMTP_ERR_INVALID_ARG
    assert call(sl=_kv(**CONTIG, batch=3)) == W.WMTP_ERR_INVALID_ARG
    assert call(max_slots=0) == W.WMTP_ERR_INVALID_ARG
    assert call(max_slots=65) == W.WMTP_ERR_INVALID_ARG
    assert call(q=None) == W.WMTP_ERR_INVALID_ARG
    assert call(hq=7) == W.WMTP_ERR_INVALID_ARG
    assert call(ws=None) == W.WMTP_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == W.WMTP_ERR_WORKSPACE


def test_fused_steps_rejected_before_launch(lib):
    L = W.lib()
    win = lambda r=_kv(), kn=FAKE, vn=FAKE, ws_bytes=1 << 30: L.wmtp_draft_step_windowed(
        ctypes.byref(r), kn, vn, FAKE, 8, 0.1, FAKE, None, FAKE, ws_bytes, None)
    full = lambda c=_kv(**CONTIG), kn=FAKE, bound=10: L.wmtp_draft_step_full(
        ctypes.byref(c), kn, FAKE, FAKE, 8, 0.1, bound, FAKE, None, FAKE, 1 << 30, None)
    assert win(kn=None) == W.WMTP_ERR_INVALID_ARG
    assert win(vn=None) == W.WMTP_ERR_INVALID_ARG
    assert win(kn=FAKE + 4) == W.WMTP_ERR_INVALID_ARG
    assert win(r=_kv(**CONTIG)) == W.WMTP_ERR_INVALID_ARG
    assert win(ws_bytes=0) == W.WMTP_ERR_WORKSPACE
    assert full(c=_kv()) == W.WMTP_ERR_INVALID_ARG
    assert full(kn=None) == W.WMTP_ERR_INVALID_ARG
    assert full(bound=0) == W.WMTP_ERR_INVALID_ARG
    assert full(bound=65) == W.WMTP_ERR_INVALID_ARG


def test_verify_step_rejected_before_launch(lib):
    L = W.lib()
    call = lambda c=_kv(**CONTIG), kn=FAKE, m=4, bound=10: L.wmtp_verify_step(
        ctypes.byref(c), kn, FAKE, FAKE, m, 8, 0.1, bound, FAKE, None, FAKE, 1 << 30, None)
    assert call(c=_kv()) == W.WMTP_ERR_INVALID_ARG
    assert call(kn=None) == W.WMTP_ERR_INVALID_ARG
    assert call(m=0) == W.WMTP_ERR_INVALID_ARG
    assert call(m=17) == W.WMTP_ERR_INVALID_ARG
    assert call(bound=65) == W.WMTP_ERR_INVALID_ARG


def test_grid_limits_rejected_before_launch(lib):
    assert _append(_kv(batch=65536)) == W.WMTP_ERR_INVALID_ARG
    # 40000 sequences x 2 KV heads = 80000 grid rows for an attention call
    assert _windowed(_kv(batch=40000)) == W.WMTP_ERR_INVALID_ARG
    assert W.lib().wmtp_attn_workspace_bytes(40000, 8, 2, 128, 1, 20) == 0


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_public_headers_compile(lang, tmp_path):
    """The headers stand alone for C and C++ callers (they declare only plain types)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    src.write_text('#include "wmtp.h"\n#include "wmtp_probe.h"\n'
                   'int main(void) { wmtp_kv kv; (void)kv; return wmtp_status_string(0) == 0; }\n')
    r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", "-I", inc, str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


# ------------------------------------------------------------------------------------------
# the binding's cached cache descriptor (host logic; stand-in device tensors, no GPU)
# ------------------------------------------------------------------------------------------
class _DeviceTensor:
    """Stands in for a dense device tensor: the binding reads only these attributes."""

    def __init__(self, numel, elem_bytes, addr=FAKE, cuda=True, dense=True):
        self._n, self._eb, self._addr = numel, elem_bytes, addr
        self.is_cuda = cuda
        self._dense = dense

    def is_contiguous(self):
        return self._dense

    def data_ptr(self):
        return self._addr

    def numel(self):
        return self._n

    def element_size(self):
        return self._eb


def _cache(batch=2, Hkv=2, d=128, cap=20, k=None):
    rows = batch * Hkv * cap * d
    return W.KVCache(k or _DeviceTensor(rows, 2), _DeviceTensor(rows, 2),
                     _DeviceTensor(batch * cap, 4), _DeviceTensor(batch, 4), batch, Hkv, d, cap,
                     4, 16, W.WMTP_BF16)


def test_cache_descriptor_is_built_once_and_rebuilt_after_a_field_changes():
    c = _cache()
    d1 = c.desc()
    assert c.desc() is d1  # reused while nothing changed
    assert (d1.k, d1.batch, d1.capacity, d1.window) == (FAKE, 2, 20, 16)
    c.k = _DeviceTensor(2 * 2 * 20 * 128, 2, addr=FAKE + 4096)
    d2 = c.desc()
    assert d2 is not d1 and d2.k == FAKE + 4096
    c.window = 8
    assert c.desc().window == 8


def test_cache_descriptor_checks_the_cache_tensors():
    with pytest.raises(ValueError, match="cache.k"):
        _cache(k=_DeviceTensor(2 * 2 * 20 * 128 - 1, 2)).desc()  # one element short
    with pytest.raises(ValueError, match="host tensor"):
        _cache(k=_DeviceTensor(2 * 2 * 20 * 128, 2, cuda=False)).desc()
    with pytest.raises(ValueError, match="dense"):
        _cache(k=_DeviceTensor(2 * 2 * 20 * 128, 2, dense=False)).desc()
    c = _cache()
    c.desc()
    c.seq_len = _DeviceTensor(1, 4)  # fewer lengths than sequences: refused at the rebuild
    with pytest.raises(ValueError, match="seq_len"):
        c.desc()


def test_noalloc_step_arguments_rejected_before_launch(lib):
    """The allocation-free windowed step validates like the workspace step, and refuses a step
    whose partials exceed its static scratch, before looking up the scratch or launching."""
    L = W.lib()
    call = lambda desc, k_new=FAKE, v_new=FAKE, q=FAKE, hq=8: L.wmtp_draft_step_windowed_noalloc(
        desc, k_new, v_new, q, hq, 0.1, FAKE, None, None)
    assert call(None) == W.WMTP_ERR_INVALID_ARG
    assert call(ctypes.byref(_kv(window=0, sink=20))) == W.WMTP_ERR_INVALID_ARG  # not a ring
    assert call(ctypes.byref(_kv()), k_new=None) == W.WMTP_ERR_INVALID_ARG
    assert call(ctypes.byref(_kv(head_dim=96))) == W.WMTP_ERR_UNSUPPORTED
    assert call(ctypes.byref(_kv()), hq=7) == W.WMTP_ERR_INVALID_ARG
    # 2048 (sequence, KV head) pairs need at least one 16 KB partial each: 32 MB of partials
    big = _kv(batch=1024, n_kv_heads=2, head_dim=256, capacity=260, sink=4, window=256)
    need = L.wmtp_attn_workspace_bytes(1024, 32, 2, 256, 1, 260)
    assert need > 16 << 20
    assert call(ctypes.byref(big), hq=32) == W.WMTP_ERR_WORKSPACE
