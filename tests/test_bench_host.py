"""The benchmark's host-side contract (CPU only): it refuses more than one GPU with a message, and
it reports profiler traffic only while the attention source is the one the counters measured."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_has_the_fields_the_benchmark_reads():
    text = open(bench.TRAFFIC_SUMMARY).read()
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l)
    assert len(fields["attn_source_sha256"].strip()) == 64
    for kind in ("full", "verify", "windowed"):
        assert int(fields[f"traffic_bytes_per_launch.{kind}"]) > 0
        # reads stay within 5% of the algorithmic bytes (no wasted re-reads)
        assert 1.0 <= float(fields[f"read_over_algorithmic.{kind}"]) <= 1.05
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text


def test_traffic_is_reported_only_for_the_measured_source(monkeypatch):
    text = open(bench.TRAFFIC_SUMMARY).read()
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l)
    measured = fields["attn_source_sha256"].strip()
    monkeypatch.setattr(bench, "attn_source_hash", lambda: measured)
    assert bench.measured_traffic("full") == int(fields["traffic_bytes_per_launch.full"])
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("full") is None
