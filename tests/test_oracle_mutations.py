"""The oracle's pins catch planted mistakes (CPU only).

Each case copies the oracle package into a temporary directory, plants one plausible mistake in
the copy (its C arithmetic or its Python position sets, ring model or accept rule), and runs the
pin suite (tests/test_oracle_pins.py) against the copy in a fresh interpreter: at least one pin
must fail. The unmodified copy must pass the same run, so a failure is the mistake's doing. The
committed oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, file in the oracle package, text, replacement, occurrences the text must have)
MUTATIONS = [
    ("score scale dropped", "wmtp_oracle.c",
     "s[j] = scale * dot;", "s[j] = dot;", 1),
    ("lse without the max", "wmtp_oracle.c",
     "lse[pr->out_off / d] = M + log(Z);", "lse[pr->out_off / d] = log(Z);", 1),
    ("scores taken against V", "wmtp_oracle.c",
     "dot += qd[i] * load_elem(k, dtype_kv, base + i);",
     "dot += qd[i] * load_elem(v, dtype_kv, base + i);", 1),
    ("output not normalised", "wmtp_oracle.c",
     "for (int32_t i = 0; i < d; ++i) o[i] /= Z;", "", 1),
    ("bf16 decoded one bit off", "wmtp_oracle.c",
     "((const uint16_t*)base)[i] << 16;", "((const uint16_t*)base)[i] << 15;", 1),
    ("last row of every run dropped", "wmtp_oracle.c",
     "r < pr->count[run]; ++r, ++j)", "r < pr->count[run] - 1; ++r, ++j)", 2),
    ("softmax in base 2", "wmtp_oracle.c",
     "double w = exp(s[j] - M);", "double w = exp2(s[j] - M);", 1),
    ("window one short", "__init__.py",
     "win_start = max(sink_stop, n - W)", "win_start = max(sink_stop, n - W + 1)", 1),
    ("one sink short", "__init__.py",
     "sink_stop = min(S, n)", "sink_stop = min(max(S - 1, 0), n)", 1),
    ("candidate does not see itself", "__init__.py",
     "return [(0, max(0, n - m + j + 1))]", "return [(0, max(0, n - m + j))]", 1),
    ("GQA heads interleaved", "__init__.py",
     "h = hq // G", "h = hq % Hkv", 1),
    ("ring slot without the sink offset", "__init__.py",
     "S + (p - S) % W", "S + p % W", 2),
    ("ring keeps the oldest writer", "__init__.py",
     "np.maximum.at(self.tags[b], s, p)", "np.minimum.at(self.tags[b], s, p)", 1),
    ("rollback leaves tags in place", "__init__.py",
     "self.tags[b, ring_slot(p, self.S, self.Wp)] = -1",
     "self.tags[b, ring_slot(p, self.S, self.Wp)] += 0", 1),
    ("rollback clamped to the slack alone", "__init__.py",
     "while d > 0 and not self.exact_after(b, d):", "while False:", 1),
    ("ties go to the highest index", "__init__.py",
     "choice = np.argmax(logits, axis=2).astype(np.int64)",
     "choice = (logits.shape[2] - 1 - np.argmax(logits[:, :, ::-1], axis=2)).astype(np.int64)", 1),
    ("newest memory slot dropped", "__init__.py",
     "SLOT_BASE + max(0, n_slots))]", "SLOT_BASE + max(0, n_slots - 1))]", 1),
]

RUNNER = """
import importlib.util, sys
pkg = sys.argv[1]
spec = importlib.util.spec_from_file_location("oracle", pkg + "/__init__.py",
                                              submodule_search_locations=[pkg])
mod = importlib.util.module_from_spec(spec)
sys.modules["oracle"] = mod
spec.loader.exec_module(mod)
mod.build()
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", sys.argv[2]]))
"""


def _copy_oracle(dst):
    pkg = os.path.join(dst, "oracle")
    os.makedirs(pkg)
    for f in ("__init__.py", "wmtp_oracle.c"):
        shutil.copy(os.path.join(ORACLE, f), os.path.join(pkg, f))
    return pkg


def _run_pins(pkg):
    env = dict(os.environ, OMP_NUM_THREADS="2")
    env.pop("WMTP_ORACLE_LIB", None)  # the copy loads the library it builds from its own source
    return subprocess.run([sys.executable, "-c", RUNNER, pkg, PINS], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    r = _run_pins(_copy_oracle(str(tmp_path)))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,fname,old,new,count", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, fname, old, new, count):
    pkg = _copy_oracle(str(tmp_path))
    path = os.path.join(pkg, fname)
    src = open(path).read()
    assert src.count(old) == count, f"{name}: the oracle no longer reads as the mutation expects"
    open(path, "w").write(src.replace(old, new))
    r = _run_pins(pkg)
    # pytest's status 1 = tests ran and at least one failed (not a crash or a collection error)
    assert r.returncode == 1, f"{name}: no pin failed\n" + r.stdout[-2000:] + r.stderr[-2000:]
