"""Float64 CPU oracle for Windowed-MTP draft attention, full draft attention, verification
attention and the compact ring buffer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product path (``draft_attention_amd``) never does, and
this package never imports the product path. The two share no code.

Everything here restates the Windowed-MTP abstract (thelatestinai.com/papers/2607.21535; the same
text appears on the khansong-paper-with-me page) in plain code:

* the native MTP draft head attends over the entire KV cache at every draft step (abstract,
  third sentence) -- :func:`full_positions`;
* Windowed-MTP gives the draft's attention a StreamingLLM-style sliding window plus attention
  sinks, and leaves full-attention verification intact (abstract, fifth sentence) --
  :func:`windowed_positions`, :func:`verify_positions`;
* the draft KV that is never read is reclaimed by a compact ring buffer (abstract, last sentence)
  -- :func:`ring_slot`, :class:`RingModel`.

The pages give no formula, no layout and no values for S, W or the slot map. The readings taken
here (listed with reasons in the design notes of the repository):

* sinks are the first S positions of the sequence, 0..S-1;
* each draft step appends its own K/V before attending, so the window is the last W of the n
  cached positions and includes the current token;
* sink and window sets are united with each position taken once (so S + W >= n gives full
  attention);
* GQA: query head hq reads KV head hq // G with G = Hq / Hkv;
* ring slot of position p: p for p < S, else S + (p - S) mod W (the first window token lands in
  slot S); a contiguous cache is the same map with S = capacity, W = 0;
* a ring may carry ``slack`` extra window slots (positions wrap over W + slack slots, the draft
  still attends the last W): up to ``slack`` newest tokens can then be discarded after a
  rejection, the MASW page's rollback of speculative local KV (section 4.3), read as
  "restore exactly the state before the rejected tokens were appended";
* greedy acceptance: draft token i is kept while it equals the target's argmax at row i (lowest
  index on ties); the target's argmax at the first rejected row is the next token;
* MASW working memory (MASW page, section 4.1): sinks, the exact local window and every memory
  slot materialised so far; slot rows are given (the adaptor that makes them is out of scope);
* verification query j of m (the candidates sit at positions n-m .. n-1) attends positions
  0 .. n-m+j, its own included;
* outputs and lse are float64 here; lse uses the natural log; an empty set gives o = 0 and
  lse = -inf.

The arithmetic of each attention problem is in ``wmtp_oracle.c`` (two-pass softmax in float64);
this module decides which rows each problem attends.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wmtp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# another build of wmtp_oracle.c to load instead (the sanitizer run of the CPU tests sets it)
_LIB_OVERRIDE = os.environ.get("WMTP_ORACLE_LIB")

F32, BF16, F64 = 0, 1, 2

Range = Tuple[int, int]  # half-open [start, stop)


# --------------------------------------------------------------------------------------------
# build / load of the C core
# --------------------------------------------------------------------------------------------
def build(verbose: bool = False, out: str = _LIB_PATH, flags: Sequence[str] = ()) -> str:
    """Compile ``wmtp_oracle.c`` into ``liboracle.so`` with gcc (plain -O2, OpenMP, IEEE).
    ``out`` and ``flags`` (extra gcc flags, e.g. sanitizers) serve other builds of the source."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *flags, _SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_RUNS = 4  # position runs per problem (ORACLE_RUNS in wmtp_oracle.c)


class _Problem(ctypes.Structure):
    _fields_ = [("q_off", ctypes.c_int64), ("kv_off", ctypes.c_int64 * _RUNS),
                ("count", ctypes.c_int64 * _RUNS), ("row_stride", ctypes.c_int64),
                ("out_off", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
        lib.wmtp_oracle_attention.restype = ctypes.c_int
        lib.wmtp_oracle_attention.argtypes = [
            ctypes.c_int64, ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        lib.wmtp_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().wmtp_oracle_max_threads())


# --------------------------------------------------------------------------------------------
# which positions each problem attends
# --------------------------------------------------------------------------------------------
def full_positions(n: int) -> List[Range]:
    """Native draft head: every cached position 0..n-1 (abstract, third sentence)."""
    return [(0, max(0, n))]


def windowed_positions(n: int, S: int, W: int) -> List[Range]:
    """Windowed-MTP draft head: attention sinks {p < S} united with the sliding window of the
    last W cached positions {n-W <= p < n} (abstract, fifth sentence), each position once."""
    if W < 1 or S < 0:
        raise ValueError("windowed attention needs W >= 1 and S >= 0")
    n = max(0, n)
    sink_stop = min(S, n)
    win_start = max(sink_stop, n - W)
    return [(0, sink_stop), (win_start, n)]


def verify_positions(n: int, m: int, j: int) -> List[Range]:
    """Full-attention verification (abstract, fifth sentence): the m candidates occupy positions
    n-m .. n-1 and candidate j sees the whole prefix plus candidates 0..j."""
    return [(0, max(0, n - m + j + 1))]


def dropped_fraction(n: int, S: int, W: int) -> float:
    """Share of the n cached draft KV entries that the windowed draft never reads."""
    kept = sum(b - a for a, b in windowed_positions(n, S, W))
    return 1.0 - kept / n


# --------------------------------------------------------------------------------------------
# the compact ring buffer (abstract, last sentence)
# --------------------------------------------------------------------------------------------
def ring_slot(p, S: int, W: int):
    """Slot of logical position p: sinks are pinned, window positions wrap over W slots.
    Works on Python ints and numpy integer arrays."""
    if W == 0:
        return p
    if isinstance(p, np.ndarray):
        return np.where(p < S, p, S + (p - S) % W)
    return p if p < S else S + (p - S) % W


class RingModel:
    """Host simulation of every append into per-sequence ring buffers of S + W + slack slots.

    ``tags[b, s]`` is the logical position held in slot s of sequence b (-1: never written or
    discarded), ``n[b]`` the number of tokens present. Window positions wrap over W + slack slots
    (slack = 0 is the compact ring of the abstract's last sentence); the draft attends the sinks and
    the last W positions only, so up to ``slack`` speculative tokens can be discarded again
    (:meth:`rollback`) as long as no position the remaining window needs has been overwritten
    (after earlier rollbacks, fewer: :meth:`exact_after`). Appends are
    applied token by token in position order, so a later token always overwrites an earlier one in
    the same slot.
    """

    def __init__(self, batch: int, S: int, W: int, slack: int = 0):
        if slack < 0:
            raise ValueError("slack must be >= 0")
        self.S, self.W, self.slack = S, W, slack
        self.Wp = W + slack  # window slots
        self.tags = np.full((batch, S + self.Wp), -1, dtype=np.int64)
        self.n = np.zeros(batch, dtype=np.int64)

    def append(self, b: int, count: int) -> None:
        if count <= 0:
            return
        p = np.arange(self.n[b], self.n[b] + count, dtype=np.int64)
        s = ring_slot(p, self.S, self.Wp)
        # positions increase, so "last writer wins" is the per-slot maximum over what is there now
        # (a discarded slot holds -1)
        np.maximum.at(self.tags[b], s, p)
        self.n[b] += count

    def exact_after(self, b: int, d: int) -> bool:
        """Whether discarding the newest d tokens leaves an exact ring: every position that a
        windowed draft step attends with n - d tokens present (the sinks and the last W) is still
        held in its slot. A slot is overwritten by the position W + slack later, so after earlier
        rollbacks a later append may already have taken a slot that a deeper rollback would need
        again."""
        if self.W < 1:
            raise ValueError("only a ring (W >= 1) overwrites slots")
        n = int(self.n[b]) - d
        for a, c in windowed_positions(n, self.S, self.W):
            for p in range(a, c):
                if self.tags[b, ring_slot(p, self.S, self.Wp)] != p:
                    return False
        return True

    def max_rollback(self, b: int) -> int:
        """The largest number of newest tokens that can be discarded exactly: at most the slack,
        and only as deep as :meth:`exact_after` allows (all of them for a contiguous cache, W = 0,
        which overwrites nothing)."""
        return self._clamp(b, int(self.n[b]))

    def _clamp(self, b: int, count: int) -> int:
        n = int(self.n[b])
        if self.W == 0:
            return max(0, min(count, n))
        d = max(0, min(count, n, self.slack))
        while d > 0 and not self.exact_after(b, d):
            d -= 1
        return d

    def rollback(self, b: int, count: int) -> int:
        """Discard the newest tokens: the largest d <= count (and <= the slack) that leaves an
        exact ring (:meth:`exact_after`). Their slots are marked empty and n shrinks. Returns d."""
        d = self._clamp(b, int(count))
        if d:
            p = np.arange(self.n[b] - d, self.n[b], dtype=np.int64)
            self.tags[b, ring_slot(p, self.S, self.Wp)] = -1
            self.n[b] -= d
        return d

    def occupied_slots(self, b: int) -> np.ndarray:
        return np.nonzero(self.tags[b] >= 0)[0]

    def attended_slots(self, b: int) -> np.ndarray:
        """Slots holding the positions a windowed draft step attends (sinks + last W)."""
        n = int(self.n[b])
        pos = np.concatenate([np.arange(a, c, dtype=np.int64)
                              for a, c in windowed_positions(n, self.S, self.W)])
        slots = ring_slot(pos, self.S, self.Wp)
        if not np.array_equal(self.tags[b, slots], pos):
            raise AssertionError("ring model lost an attended position")
        return np.sort(slots)


def greedy_accept(target_logits: np.ndarray, draft_tokens: np.ndarray):
    """Greedy verification of k draft tokens (the standard accept/reject rule under greedy
    decoding; MASW page, section 1 and 4.3: the target keeps its accept/reject rule and rejected
    speculative draft KV is discarded).

    ``target_logits`` is ``[B][k+1][V]``: row i scores the token that follows the prefix plus the
    first i drafts. Draft token i is accepted while it equals the target's choice (argmax; the
    lowest index on ties) at row i and every earlier draft was accepted. The target's choice at the
    first rejected row (or at row k when all are accepted) is the next token. Returns
    ``(choice [B][k+1], n_accept [B], next_token [B], n_drop [B] = k - n_accept)``."""
    logits = np.asarray(target_logits)
    B, k1, _ = logits.shape
    k = k1 - 1
    draft = np.asarray(draft_tokens).reshape(B, k)
    choice = np.argmax(logits, axis=2).astype(np.int64)  # first maximum on ties
    n_accept = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = 0
        while a < k and draft[b, a] == choice[b, a]:
            a += 1
        n_accept[b] = a
    next_token = choice[np.arange(B), n_accept]
    return choice, n_accept, next_token, k - n_accept


# --------------------------------------------------------------------------------------------
# KV rows addressed by logical position
# --------------------------------------------------------------------------------------------
@dataclass
class LogicalKV:
    """K and V rows of B sequences, ``[B][Hkv][R][d]``, together with the logical positions they
    hold. ``segments[b]`` lists ``(first_position, first_row, count)`` runs; a full contiguous
    sequence is the single run ``(0, 0, R)``. ``k`` and ``v`` are float32, float64 or uint16
    (bf16 bit patterns, ``dtype=BF16``)."""

    k: np.ndarray
    v: np.ndarray
    dtype: int
    segments: Sequence[Sequence[Tuple[int, int, int]]]

    @property
    def shape(self):
        return self.k.shape

    def row_run(self, b: int, p0: int, p1: int) -> Tuple[int, int]:
        """(first_row, count) of the rows holding positions [p0, p1); they must be one run."""
        if p1 <= p0:
            return 0, 0
        for first_pos, first_row, count in self.segments[b]:
            if first_pos <= p0 and p1 <= first_pos + count:
                return first_row + (p0 - first_pos), p1 - p0
        raise KeyError(f"positions [{p0},{p1}) of sequence {b} are not held as one run")

    def row_indices(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Row holding each position of sequence b (KeyError if one is not held)."""
        positions = np.asarray(positions, dtype=np.int64)
        rows = np.full(positions.shape, -1, dtype=np.int64)
        for first_pos, first_row, count in self.segments[b]:
            inside = (positions >= first_pos) & (positions < first_pos + count)
            rows[inside] = first_row + (positions[inside] - first_pos)
        if np.any(rows < 0):
            raise KeyError(f"positions {positions[rows < 0][:4]} of sequence {b} are not held")
        return rows

    def rows_of_positions(self, b: int, h: int, positions: np.ndarray, which: str = "k"):
        arr = self.k if which == "k" else self.v
        return arr[b, h, self.row_indices(b, positions)]


def contiguous_kv(k: np.ndarray, v: np.ndarray, dtype: int) -> LogicalKV:
    """K/V ``[B][Hkv][n][d]`` holding positions 0..n-1 of every sequence."""
    B, _, n, _ = k.shape
    return LogicalKV(k, v, dtype, [[(0, 0, n)] for _ in range(B)])


def _np_dtype_code(a: np.ndarray, declared: int) -> int:
    if declared == BF16:
        assert a.dtype == np.uint16, "bf16 arrays are passed as uint16 bit patterns"
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported array dtype {a.dtype}")


# --------------------------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------------------------
def attention(q: np.ndarray, q_dtype: int, kv: LogicalKV, sets, scale: float,
              nthreads: int = 0):
    """Softmax attention of every query row over its own set of positions.

    ``q`` is ``[B][m][Hq][d]``; ``sets[b][j]`` is the list of position ranges that query token j
    of sequence b attends (shared by its Hq heads); query head hq reads KV head hq // G.
    Returns ``(out [B][m][Hq][d] float64, lse [B][m][Hq] float64)``.
    """
    q = np.ascontiguousarray(q)
    B, m, Hq, d = q.shape
    kb, Hkv, R, dk = kv.k.shape
    assert kb == B and dk == d and Hq % Hkv == 0
    G = Hq // Hkv
    k = np.ascontiguousarray(kv.k)
    v = np.ascontiguousarray(kv.v)
    qcode = _np_dtype_code(q, q_dtype)
    kvcode = _np_dtype_code(k, kv.dtype)
    probs = (_Problem * (B * m * Hq))()
    i = 0
    for b in range(B):
        for j in range(m):
            ranges = [r for r in sets[b][j] if r[1] > r[0]]
            if len(ranges) > _RUNS:
                raise ValueError(f"at most {_RUNS} position ranges per problem")
            for hq in range(Hq):
                h = hq // G
                pr = probs[i]
                pr.q_off = ((b * m + j) * Hq + hq) * d
                pr.row_stride = d
                pr.out_off = ((b * m + j) * Hq + hq) * d
                for run in range(_RUNS):
                    if run < len(ranges):
                        r0, cnt = kv.row_run(b, ranges[run][0], ranges[run][1])
                        pr.kv_off[run] = ((b * Hkv + h) * R + r0) * d
                        pr.count[run] = cnt
                    else:
                        pr.kv_off[run] = 0
                        pr.count[run] = 0
                i += 1
    out = np.zeros((B, m, Hq, d), dtype=np.float64)
    lse = np.zeros((B, m, Hq), dtype=np.float64)
    rc = _load().wmtp_oracle_attention(
        len(probs), probs, d, qcode, kvcode, q.ctypes.data, k.ctypes.data, v.ctypes.data,
        float(scale), out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, lse


def draft_full(q, q_dtype, kv: LogicalKV, n: Sequence[int], scale: float, nthreads: int = 0):
    """Native draft step: one query token per sequence attends positions 0..n_b-1.
    ``q`` is ``[B][1][Hq][d]``."""
    sets = [[full_positions(int(n[b]))] for b in range(q.shape[0])]
    return attention(q, q_dtype, kv, sets, scale, nthreads)


def draft_windowed(q, q_dtype, kv: LogicalKV, n: Sequence[int], S: int, W: int, scale: float,
                   nthreads: int = 0):
    """Windowed-MTP draft step over the logical sequence: sinks plus the last W positions."""
    sets = [[windowed_positions(int(n[b]), S, W)] for b in range(q.shape[0])]
    return attention(q, q_dtype, kv, sets, scale, nthreads)


SLOT_BASE = 1 << 40  # label of memory slot j in a MASW working set: SLOT_BASE + j


def masw_kv(kv: LogicalKV, slots_k: np.ndarray, slots_v: np.ndarray) -> LogicalKV:
    """The raw rows of ``kv`` followed by memory-slot rows ``[B][Hkv][M][d]`` (same dtype), slot j
    labelled with position SLOT_BASE + j."""
    B, Hkv, R, d = kv.k.shape
    M = slots_k.shape[2]
    k = np.concatenate([kv.k, slots_k.astype(kv.k.dtype)], axis=2)
    v = np.concatenate([kv.v, slots_v.astype(kv.v.dtype)], axis=2)
    segments = [list(kv.segments[b]) + [(SLOT_BASE, R, M)] for b in range(B)]
    return LogicalKV(k, v, kv.dtype, segments)


def masw_positions(n: int, S: int, W: int, n_slots: int) -> List[Range]:
    """MASW working memory (MASW page, section 4.1): the sink tokens, the exact local window and
    the memory slots materialised so far, each once."""
    return windowed_positions(n, S, W) + [(SLOT_BASE, SLOT_BASE + max(0, n_slots))]


def draft_masw(q, q_dtype, kv: LogicalKV, n: Sequence[int], S: int, W: int, slots_k, slots_v,
               n_slots: Sequence[int], scale: float, nthreads: int = 0):
    """MASW-style draft step: one query token per sequence attends the sinks and the last W of
    its n_b raw positions plus its first n_slots[b] memory slots (the slot rows are inputs; how
    a slot is materialised from history is the adaptor's business and not computed here)."""
    both = masw_kv(kv, slots_k, slots_v)
    sets = [[masw_positions(int(n[b]), S, W, int(n_slots[b]))] for b in range(q.shape[0])]
    return attention(q, q_dtype, both, sets, scale, nthreads)


def verify(q, q_dtype, kv: LogicalKV, n: Sequence[int], scale: float, nthreads: int = 0):
    """Verification of m candidates (the last m of the n cached positions), causal among them.
    ``q`` is ``[B][m][Hq][d]``."""
    m = q.shape[1]
    sets = [[verify_positions(int(n[b]), m, j) for j in range(m)] for b in range(q.shape[0])]
    return attention(q, q_dtype, kv, sets, scale, nthreads)


def ring_attention(q, q_dtype, ring_k, ring_v, kv_dtype: int, tags: np.ndarray, scale: float,
                   nthreads: int = 0, slots=None):
    """Attention over slots of ring buffers ``[B][Hkv][slots][d]`` as the hardware layout holds
    them (slots in slot order, whatever positions they carry): the occupied slots
    (``tags[b, s] >= 0``), or the slots ``slots[b]`` when given (a ring with slack also holds
    positions older than the window)."""
    B = q.shape[0]
    nslots = ring_k.shape[2]
    kv = LogicalKV(ring_k, ring_v, kv_dtype, [[(0, 0, nslots)] for _ in range(B)])
    sets = []
    for b in range(B):
        occ = np.nonzero(tags[b] >= 0)[0] if slots is None else np.sort(np.asarray(slots[b]))
        runs: List[Range] = []
        for s in occ:
            if runs and runs[-1][1] == s:
                runs[-1] = (runs[-1][0], s + 1)
            else:
                runs.append((int(s), int(s) + 1))
        sets.append([runs])
    return attention(q, q_dtype, kv, sets, scale, nthreads)


def ring_expected(model: RingModel, kv: LogicalKV):
    """Expected ring contents for the positions recorded in ``model.tags``: K and V arrays
    ``[B][Hkv][slots][d]`` (rows of empty slots are zero) gathered from the logical sequence."""
    B, Hkv, _, d = kv.k.shape
    nslots = model.tags.shape[1]
    rk = np.zeros((B, Hkv, nslots, d), dtype=kv.k.dtype)
    rv = np.zeros((B, Hkv, nslots, d), dtype=kv.v.dtype)
    for b in range(B):
        occ = model.occupied_slots(b)
        pos = model.tags[b, occ]
        for h in range(Hkv):
            rk[b, h, occ] = kv.rows_of_positions(b, h, pos, "k")
            rv[b, h, occ] = kv.rows_of_positions(b, h, pos, "v")
    return rk, rv
