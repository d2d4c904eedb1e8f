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


def test_trace_summary_has_the_kernel_times_the_gates_read():
    text = open(bench.TRACE_SUMMARY).read()
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l)
    traffic = dict(l.split(": ", 1) for l in open(bench.TRAFFIC_SUMMARY).read().splitlines()
                   if ": " in l)
    # both summaries were taken from the same attention source
    assert fields["attn_source_sha256"].strip() == traffic["attn_source_sha256"].strip()
    for kind in ("windowed", "full", "verify"):
        assert float(fields[f"kernel_us.{kind}.main"]) > 0
        assert float(fields[f"kernel_us.{kind}.merge"]) > 0
        assert int(traffic[f"traffic_bytes_per_launch.{kind}_merge"]) > 0
    assert "rocprofv3 --kernel-trace" in text


def test_gate_entry_reads_the_profiles_only_for_their_source(monkeypatch):
    text = open(bench.TRACE_SUMMARY).read()
    measured = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l)["attn_source_sha256"].strip()
    monkeypatch.setattr(bench, "attn_source_hash", lambda: measured)
    nbytes = 1_073_750_000
    g = bench.gate("verify", nbytes, 200.0, 190.0, None, "verify")
    k_us = bench.traced_kernel_us("verify.main")
    assert g["kernel_us_trace"] == k_us and g["merge_us_trace"] == bench.traced_kernel_us("verify.merge")
    assert abs(g["call_frac"] - nbytes / 200e-6 / 1e9 / bench.PEAK_HBM_GBS) < 1e-4
    assert g["pass_call"] == (g["call_frac"] >= 0.75)
    assert g["traffic_bytes"] == bench.measured_traffic("verify") + bench.measured_traffic("verify_merge")
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    g = bench.gate("verify", nbytes, 200.0, 190.0, None, "verify")
    assert g["kernel_us_trace"] is None and g["traffic_bytes"] is None and g["pass_kernel"] is None


def test_host_cpu_reports_the_usable_cores():
    h = bench.host_cpu()
    assert h["usable_cpus"] >= 1 and h["logical_cpus"] >= h["usable_cpus"]
