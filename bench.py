"""Benchmark of the Windowed-MTP draft-attention hot path on one MI355X.

One step = one decode iteration at a 1,048,576-token context:
  * k = 5 draft steps on the million-token draft shapes (32 query / 2 KV heads, head_dim 256, bf16,
    S = 4 sinks, W = 4096 window), each done in both forms side by side:
      - Windowed-MTP: append the draft token to the compact ring buffer, attend sinks + window;
      - native MTP:   append the draft token to the contiguous cache, attend all n tokens;
  * the target's verification of k+1 = 4 candidates on the verify shapes (32 query / 2 KV heads,
    head_dim 128, bf16): append the candidates to the target cache, causal full attention.
Every kernel is the HIP library's, called through its C ABI; inputs are seeded synthetic draws
already resident in HBM when timing starts.

Prints ONE JSON line. `value` is the whole step's algorithmic HBM bytes / step time (GB/s).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--graph]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth
PROBE_BYTES = 2 << 30  # read-probe buffer (also the source of the backlog reads)
FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache
SWEEP_L = (4096, 16384, 65536, 131072, 262144, 524288, 1048576)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the context-length sweep of single calls")
    ap.add_argument("--no-composite", action="store_true",
                    help="skip the speculative decode-iteration composite")
    ap.add_argument("--graph", action="store_true",
                    help="replay each phase of the iteration as a captured HIP graph instead of "
                         "launching every call from Python")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (reference for "
                         "scaling the HBM byte counters of a profiler) and exit")
    return ap.parse_args()


def copy_calibration():
    import torch

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_decode_step_L1M.txt")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "kernel_trace_decode_step_L1M.txt")
GATE_FRAC = 0.75  # each gated read must reach this share of the HBM peak
CLOCK_WARM_S = 0.06  # sustained load before measuring: the GPU's clocks ramp up over ~25 ms


def attn_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in ("attn.hip", "wmtp_internal.h"):
        with open(os.path.join(ROOT, "draft_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def summary_fields(path: str):
    """The `key: value` lines of a committed profile summary, or None when the attention source
    changed since its numbers were taken (its recorded source hash differs)."""
    try:
        with open(path) as fh:
            fields = dict(l.split(": ", 1) for l in fh.read().splitlines() if ": " in l)
    except OSError:
        return None
    if fields.get("attn_source_sha256", "").strip() != attn_source_hash():
        return None
    return {k.strip(): v.strip() for k, v in fields.items()}


def measured_traffic(kind: str):
    """HBM bytes per launch (profiler FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading)
    from the committed summary, or None when the attention source changed since it was taken."""
    fields = summary_fields(TRAFFIC_SUMMARY)
    v = None if fields is None else fields.get(f"traffic_bytes_per_launch.{kind}")
    return None if v is None else int(float(v))


def traced_kernel_us(kind: str):
    """Average kernel-only duration (us) of one kernel of a call from the committed rocprofv3
    kernel trace (kind e.g. windowed.split, windowed.merge), or None when the source changed."""
    fields = summary_fields(TRACE_SUMMARY)
    v = None if fields is None else fields.get(f"kernel_us.{kind}")
    return None if v is None else float(v)


def host_cpu():
    """Model name of the host CPU and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def capture(fn):
    """A HIP graph of the work fn enqueues, captured on a side stream. (torch.cuda.graph() would
    first call torch.cuda.empty_cache(); releasing cached device memory to the driver leaves the
    long attention kernels about 5% slower for the rest of the process, so the benchmark never
    does it.)"""
    import torch

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            fn()
        finally:
            g.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    return g


def steady_graph_us(fn, calls: int, reps: int = 3) -> float:
    """Per-call time in steady state: `calls` invocations of fn in one graph, replayed back to back
    for CLOCK_WARM_S (the GPU's clocks ramp up over the first ~25 ms of sustained load after any
    idle time), then `reps` timed replays; the median per call."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()

    def body():
        for _ in range(calls):
            fn()
    g = capture(body)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_WARM_S:
        g.replay()
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(1000.0 * e0.elapsed_time(e1) / calls)
    del g
    return sorted(per)[len(per) // 2]


def graph_us(fn, calls: int = 100, reps: int = 3) -> float:
    """Per-call time of `calls` invocations of fn captured in one HIP graph and replayed back to
    back (no host launch gaps, no event per call); the best of `reps` replays."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()

    def body():
        for _ in range(calls):
            fn()
    g = capture(body)
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, 1000.0 * e0.elapsed_time(e1) / calls)
    del g
    return best


def fill_sequence(dst, seed, tensor_id, b, p0, p1, dtype, device, chunk=1 << 17):
    """Write the seeded rows of positions [p0, p1) of sequence b into dst[:, p0:p1] (head-major)."""
    from draft_attention_amd import synth

    H, d = dst.shape[0], dst.shape[2]
    for c0 in range(p0, p1, chunk):
        c1 = min(p1, c0 + chunk)
        dst[:, c0:c1] = synth.sequence_rows(seed, tensor_id, b, c0, c1, H, d, dtype, device)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: the attention path runs on one GPU (got --gpus {args.gpus}); it has no "
              "multi-GPU form", file=sys.stderr)
        sys.exit(2)

    import torch

    from draft_attention_amd import binding as W
    from draft_attention_amd import configs, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W.lib()
    dt = torch.bfloat16
    D3, V4 = configs.MILLION, configs.VERIFY
    L, k = D3.context, D3.draft_depth
    m = V4.verify_m
    total_steps = args.warmup + args.steps
    log = lambda s: print(s, file=sys.stderr, flush=True)

    # ---------------- draft caches (million-token draft shapes)
    Hq, Hkv, d, S, Wn = D3.n_q_heads, D3.n_kv_heads, D3.head_dim, D3.sink, D3.window
    cap = L + k * total_steps + 16 + COMPOSITE_MARGIN
    log(f"setup: contiguous draft cache {Hkv}x{cap}x{d} bf16, ring {S}+{Wn}")
    full = W.KVCache.contiguous(1, Hkv, d, cap, dt, dev)
    fill_sequence(full.k[0], D3.seed, synth.K_ID, 0, 0, L, dt, dev)
    fill_sequence(full.v[0], D3.seed, synth.V_ID, 0, 0, L, dt, dev)
    full.seq_len.fill_(L)
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, dt, dev)
    # the ring state after L appends holds the sinks and the last W positions: append those only
    for p0, p1 in ((0, S), (L - Wn, L)):
        ring.seq_len.fill_(p0)
        kn = synth.token_rows(D3.seed, synth.K_ID, 0, p0, p1, Hkv, d, dt, dev)[None]
        vn = synth.token_rows(D3.seed, synth.V_ID, 0, p0, p1, Hkv, d, dt, dev)[None]
        W.wmtp_ring_append(ring, kn, vn, p1 - p0)
    ntok = k * total_steps
    draft_k = synth.token_rows(D3.seed, synth.K_ID, 0, L, L + ntok, Hkv, d, dt, dev)
    draft_v = synth.token_rows(D3.seed, synth.V_ID, 0, L, L + ntok, Hkv, d, dt, dev)
    draft_q = [synth.queries(D3.seed, i, 1, 1, Hq, d, dt, dev) for i in range(ntok)]
    scale3 = 1.0 / math.sqrt(d)
    ws_full = W.workspace(1, Hq, Hkv, d, 1, cap, dev)
    ws_win = W.workspace(1, Hq, Hkv, d, 1, S + Wn, dev)
    out3 = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse3 = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)

    # ---------------- target cache (verify shapes)
    Hq4, Hkv4, d4 = V4.n_q_heads, V4.n_kv_heads, V4.head_dim
    cap4 = L + m * total_steps + 16 + COMPOSITE_MARGIN
    log(f"setup: target cache {Hkv4}x{cap4}x{d4} bf16")
    tgt = W.KVCache.contiguous(1, Hkv4, d4, cap4, dt, dev)
    fill_sequence(tgt.k[0], V4.seed, synth.K_ID, 0, 0, L, dt, dev)
    fill_sequence(tgt.v[0], V4.seed, synth.V_ID, 0, 0, L, dt, dev)
    tgt.seq_len.fill_(L)
    cand_k = synth.token_rows(V4.seed, synth.K_ID, 0, L, L + m * total_steps, Hkv4, d4, dt, dev)
    cand_v = synth.token_rows(V4.seed, synth.V_ID, 0, L, L + m * total_steps, Hkv4, d4, dt, dev)
    ver_q = [synth.queries(V4.seed, i, 1, m, Hq4, d4, dt, dev) for i in range(total_steps)]
    scale4 = 1.0 / math.sqrt(d4)
    ws_ver = W.workspace(1, Hq4, Hkv4, d4, m, cap4, dev)
    out4 = torch.empty((1, m, Hq4, d4), dtype=torch.float32, device=dev)
    lse4 = torch.empty((1, m, Hq4), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # the three phases of a decode iteration, and their attention-only parts
    # a draft step appends its token and attends: one fused call (wmtp_draft_step_*)
    def win_phase(s: int, append: bool = True):
        for i in range(k):
            t = s * k + i
            if append:
                W.wmtp_draft_step_windowed(ring, draft_k[t:t + 1][None], draft_v[t:t + 1][None],
                                           draft_q[t], Hq, scale3, out3, lse3, ws_win)
            else:
                W.wmtp_draft_attn_windowed(ring, draft_q[t], Hq, scale3, out3, lse3, ws_win)

    def full_phase(s: int, append: bool = True):
        for i in range(k):
            t = s * k + i
            if append:
                W.wmtp_draft_step_full(full, draft_k[t:t + 1][None], draft_v[t:t + 1][None],
                                       draft_q[t], Hq, scale3, cap, out3, lse3, ws_full)
            else:
                W.wmtp_draft_attn_full(full, draft_q[t], Hq, scale3, cap, out3, lse3, ws_full)

    def ver_phase(s: int, append: bool = True):
        if append:  # the target appends the candidates and verifies them: one fused call
            W.wmtp_verify_step(tgt, cand_k[s * m:(s + 1) * m][None],
                               cand_v[s * m:(s + 1) * m][None], ver_q[s], m, Hq4, scale4, cap4,
                               out4, lse4, ws_ver)
        else:
            W.wmtp_verify_attn(tgt, ver_q[s], m, Hq4, scale4, cap4, out4, lse4, ws_ver)

    phases = {"win": win_phase, "full": full_phase, "ver": ver_phase}
    if not args.graph:
        # every call launched from Python: includes the host's launch latency between calls
        run = {name: (lambda f: (lambda s, append=True: f(s, append)))(f) for name, f in phases.items()}
        launch = "eager (one host launch per call)"
    else:
        # one HIP graph per phase (captured once, replayed): the kernels of a phase run back to
        # back on the GPU, as inside a serving engine's captured decode loop. Every replay
        # appends (the same token bytes) at the next positions, so caches keep growing. Graphs
        # are captured without releasing cached memory (see capture()), so replays run as fast
        # as direct launches.
        graphs = {}
        for name, f in phases.items():
            for append in (True, False):
                graphs[(name, append)] = capture(lambda f=f, append=append: f(0, append))
        run = {name: (lambda nm: (lambda s, append=True: graphs[(nm, append)].replay()))(name)
               for name in phases}
        launch = "hip-graph (one captured graph per phase, replayed)"

    # untimed clock warm-up: attention-only full-context calls (they leave the caches as they are)
    # for CLOCK_WARM_S, so the warm-up steps and the timed steps run at the clocks sustained load
    # settles at rather than ramping up from idle
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < CLOCK_WARM_S:
        run["full"](0, append=False)
        torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        for name in ("win", "full", "ver"):
            run[name](s)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ({launch})")
    rec = {"win": [], "full": [], "ver": []}
    marks = []
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.warmup, total_steps):
        e = [ev() for _ in range(4)]
        e[0].record(stream)
        run["win"](s)
        e[1].record(stream)
        run["full"](s)
        e[2].record(stream)
        run["ver"](s)
        e[3].record(stream)
        marks.append(e)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    for e in marks:
        rec["win"].append(e[0].elapsed_time(e[1]))
        rec["full"].append(e[1].elapsed_time(e[2]))
        rec["ver"].append(e[2].elapsed_time(e[3]))
    # attention alone (outside the timed steps): the same phases without the appends, each
    # enqueued behind a ~0.15 ms read of another buffer so that the host has queued every call
    # before the GPU reaches the first one (the events then bracket GPU work only)
    probe_buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device=dev)
    probe_out = torch.empty(W.WMTP_PROBE_BLOCKS, dtype=torch.int32, device=dev)
    backlog = lambda: W.wmtp_probe_read(probe_buf, probe_out, 1 << 30)
    attn_only = {"win": [], "full": [], "ver": []}
    for rep in range(max(3, args.steps // 2)):
        for name in ("win", "full", "ver"):
            e0, e1 = ev(), ev()
            backlog()
            e0.record(stream)
            run[name]((args.warmup + rep) % total_steps, append=False)
            e1.record(stream)
            torch.cuda.synchronize()
            attn_only[name].append(e0.elapsed_time(e1))
    # the same single calls graph-replayed back to back (no host launch gaps or per-call events),
    # the windowed call also cold (each call behind a 512 MiB cache flush, the flush's own time
    # subtracted), and the launch floors beside the windowed read
    log("graph-replayed single calls and launch floors")
    t_mid = args.warmup * k
    calls_of = {
        "win": lambda: W.wmtp_draft_attn_windowed(ring, draft_q[t_mid], Hq, scale3, out3, lse3, ws_win),
        "full": lambda: W.wmtp_draft_attn_full(full, draft_q[t_mid], Hq, scale3, cap, out3, lse3, ws_full),
        "ver": lambda: W.wmtp_verify_attn(tgt, ver_q[args.warmup], m, Hq4, scale4, cap4, out4, lse4, ws_ver),
    }
    call_graph_us = {"win": steady_graph_us(calls_of["win"], 400),
                     "full": steady_graph_us(calls_of["full"], 20),
                     "ver": steady_graph_us(calls_of["ver"], 40)}
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush = lambda: W.wmtp_llc_flush(flush_buf)
    flush_us = graph_us(flush, 50)
    win_cold_graph = graph_us(lambda: (flush(), calls_of["win"]()), 50) - flush_us
    tiny = torch.empty(256, dtype=torch.uint8, device=dev)
    ring_copy = torch.empty(2 * ring.k.numel() * ring.k.element_size(), dtype=torch.uint8, device=dev)
    # the windowed call's split launch: one 16-key tile per wavefront, four wavefronts per
    # workgroup, each workgroup leaving 16 rows x d float32 plus 16 (max, sum) pairs
    cdiv = lambda a, b: -(-a // b)
    win_groups = Hkv * cdiv(cdiv(S + Wn, 16), 4)
    part_bytes = 16 * d * 4 + 16 * 8
    parts_buf = torch.empty(max(win_groups, 256) * part_bytes, dtype=torch.uint8, device=dev)
    handoff_out = torch.empty(W.WMTP_PROBE_HANDOFF_BLOCKS, dtype=torch.int32, device=dev)
    handoff = lambda g: W.wmtp_probe_handoff(ring_copy, g, parts_buf, part_bytes, handoff_out)
    read_ring = lambda: W.wmtp_probe_read(ring_copy, probe_out)
    floors = {
        "one_launch_us": round(graph_us(lambda: W.wmtp_llc_flush(tiny), 200), 3),
        "two_launches_us": round(graph_us(lambda: (W.wmtp_llc_flush(tiny), W.wmtp_llc_flush(tiny)), 200), 3),
        "ring_bytes_read_one_launch_us": round(graph_us(read_ring, 200), 3),
        "ring_bytes_read_one_launch_cold_us": round(graph_us(lambda: (flush(), read_ring()), 50) - flush_us, 3),
        "handoff_skeleton_us": {str(g): round(graph_us(lambda g=g: handoff(g), 200), 3)
                                for g in (win_groups, 256)},
        "handoff_skeleton_cold_us": {str(g): round(graph_us(lambda g=g: (flush(), handoff(g)), 50) - flush_us, 3)
                                     for g in (win_groups, 256)},
        "handoff_part_bytes": part_bytes,
        "note": "graph-replayed, back to back: an (almost) empty kernel of the library "
                "(wmtp_llc_flush of 256 bytes), two of them, the read probe streaming as many "
                "bytes as the ring's K and V once, and the hand-off skeleton (wmtp_probe_handoff: "
                "the ring's bytes read by g workgroups that each write one partial of "
                "handoff_part_bytes, then 256 workgroups reading the partials back; no arithmetic) "
                "at the windowed call's own split count and at 256; *_cold: each behind a 512 MiB "
                "cache flush, the flush's own time subtracted. The windowed call is two dependent "
                "launches (split-K partials, then the merge)",
    }
    del flush_buf, ring_copy, parts_buf
    masw_res = None if args.no_composite else masw_step(
        W, synth, D3, full, ring, Hq, scale3, stream, ev, log)
    other = None if args.no_sweep else other_workloads(W, synth, configs, stream, ev, log,
                                                         cpu=not args.no_cpu_baseline)
    comp = None if args.no_composite else composite(
        W, synth, D3, V4, full, tgt, cap, cap4, stream, ev, log)
    read_ceiling = read_probe(W, probe_buf, probe_out, stream, ev)
    log(f"read probe: {read_ceiling:.1f} GB/s")
    sweep_res = None if args.no_sweep else sweep(
        W, synth, D3, full, cap, Hq, scale3, probe_buf, probe_out, stream, ev, log)
    mean = lambda v: 1000.0 * sum(v) / len(v)
    mean_us = {
        "win_step": mean(rec["win"]) / k, "full_step": mean(rec["full"]) / k,
        "ver_step": mean(rec["ver"]),
        "win_attn": mean(attn_only["win"]) / k, "full_attn": mean(attn_only["full"]) / k,
        "ver_attn": mean(attn_only["ver"]),
    }

    # algorithmic HBM bytes (K and V rows read once; q, out, lse; appends read+write the token)
    n_mid = L + k * args.warmup + (k * args.steps) // 2  # mean tokens present during the timed draft
    win_slots = S + Wn
    b_win = 2 * win_slots * Hkv * d * 2 + Hq * d * 2 + Hq * (d + 1) * 4
    b_full = 2 * n_mid * Hkv * d * 2 + Hq * d * 2 + Hq * (d + 1) * 4
    n4_mid = L + m * args.warmup + (m * args.steps) // 2 + m
    b_ver = 2 * n4_mid * Hkv4 * d4 * 2 + m * Hq4 * d4 * 2 + m * Hq4 * (d4 + 1) * 4
    b_app3 = 2 * 2 * Hkv * d * 2
    b_app4 = 2 * 2 * m * Hkv4 * d4 * 2
    step_bytes = k * (b_win + b_full + 2 * b_app3) + b_ver + b_app4
    ms_step = total_ms / args.steps
    win_cold = sweep_res["windowed_us_cold"][-1]["p50"] if sweep_res else None
    full_cold = sweep_res["full_us_cold"][-1]["p50"] if sweep_res else None
    gbs = lambda nbytes, us: nbytes / (us * 1e-6) / 1e9
    result = {
        "metric": "draft-step attn µs & HBM GB/s at 1M ctx, windowed vs full (1 GPU)",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based N(0,1) draws, resident in HBM)",
        "config": {
            "workload": "decode iteration at L=1048576: 5 draft steps (32q/2kv, d256, S4, W4096; "
                        "windowed ring and full contiguous side by side) + verify of 4 candidates "
                        "(32q/2kv, d128)",
            "context": L, "draft_depth": k, "verify_m": m, "batch": 1,
        },
        "launch": launch,
        "draft_step_us": {
            "windowed_attn": round(mean_us["win_attn"], 2),
            "windowed_attn_plus_append": round(mean_us["win_step"], 2),
            "full_attn": round(mean_us["full_attn"], 2),
            "full_attn_plus_append": round(mean_us["full_step"], 2),
            "full_over_windowed": round(mean_us["full_step"] / mean_us["win_step"], 1),
            "windowed_attn_cold_p50": win_cold,
            "full_attn_cold_p50": full_cold,
            "timing": "*_attn: the attention calls alone, back to back behind a backlog read "
                      "(warm: the windowed ring was read by the previous call); "
                      "*_plus_append: the one-call steps inside the timed decode iterations; "
                      "*_cold_p50: median single call after a cache flush (sweep at L=1048576)",
        },
        "hbm_gbs": {
            "windowed_attn": round(gbs(b_win, mean_us["win_attn"]), 1),
            "full_attn": round(gbs(b_full, mean_us["full_attn"]), 1),
            "verify_attn": round(gbs(b_ver, mean_us["ver_attn"]), 1),
            "windowed_attn_cold": None if win_cold is None else round(gbs(b_win, win_cold), 1),
        },
        "hbm_frac_of_peak": {
            "windowed_attn": round(gbs(b_win, mean_us["win_attn"]) / PEAK_HBM_GBS, 4),
            "full_attn": round(gbs(b_full, mean_us["full_attn"]) / PEAK_HBM_GBS, 4),
            "verify_attn": round(gbs(b_ver, mean_us["ver_attn"]) / PEAK_HBM_GBS, 4),
        },
        "verify_us": {"attn": round(mean_us["ver_attn"], 2),
                      "attn_plus_append": round(mean_us["ver_step"], 2)},
        "dropped_kv_fraction": round(1.0 - win_slots / n_mid, 5),
        "read_probe_gbs": round(read_ceiling, 1),
        "composite": comp,
        "other_workloads": other,
        "masw": masw_res,
        "sweep": sweep_res,
        "gates": {
            "windowed": gate("windowed draft attention (split-K kernel + LSE merge), 4100 ring "
                             "slots, 32q/2kv, d256, bf16", b_win, mean_us["win_attn"],
                             call_graph_us["win"], win_cold_graph, "windowed", floors),
            "full": gate("full-context draft attention (split-K kernel + LSE merge), L=1048576, "
                         "32q/2kv, d256, bf16", b_full, mean_us["full_attn"], call_graph_us["full"],
                         None, "full"),
            "verify": gate("verification attention m=4 (cooperative MFMA kernel + LSE merge), "
                           "L=1048576, 32q/2kv, d128, bf16", b_ver, mean_us["ver_attn"],
                           call_graph_us["ver"], None, "verify"),
            "note": "call_us: event-timed calls back to back behind a backlog read (as *_attn in "
                    "draft_step_us); call_us_graph: graph-replayed in steady state (after 60 ms of "
                    "the same calls: the clocks ramp up over ~25 ms of load after idle time), median "
                    "of 3 replays; kernel_us_trace / merge_us_trace: "
                    "kernel-only means from the committed rocprofv3 kernel trace "
                    "(profiles/kernel_trace_decode_step_L1M.txt), traffic: FETCH_SIZE + WRITE_SIZE of "
                    "both kernels (profiles/hbm_traffic_decode_step_L1M.txt), both null when the "
                    "attention source changed since they were taken; pass_*: frac >= 0.75",
        },
        "roofline": {
            "kernel": "full-context draft attention call (split-K attention + LSE merge, "
                      "back to back), L=1048576, 32q/2kv, d256, bf16",
            "bound": "hbm",
            "achieved": round(gbs(b_full, mean_us["full_attn"]), 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs(b_full, mean_us["full_attn"]) / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("full"),
            "traffic_unit": "bytes per launch (split-K kernel; null if the kernel changed since "
                            "the counters in profiles/ were taken)",
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(full, tgt, ring, draft_q, ver_q, k, m, S, Wn,
                                              scale3, scale4, step_bytes, log, other,
                                              call_graph_us)
    print(json.dumps(result), flush=True)


def gate(desc, nbytes, call_us, call_us_graph, cold_us_graph, kind, floors=None):
    """Per-kernel gate entry: the call's and the kernel's share of the HBM peak, with the traced
    kernel-only times and the measured traffic of both kernels (split-K or cooperative + merge)."""
    frac = lambda us: None if us is None else round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    k_us = traced_kernel_us(f"{kind}.main")
    m_us = traced_kernel_us(f"{kind}.merge")
    t_main, t_merge = measured_traffic(kind), measured_traffic(f"{kind}_merge")
    traffic = None if t_main is None or t_merge is None else t_main + t_merge
    entry = {
        "kernel": desc,
        "algorithmic_bytes": int(nbytes),
        "call_us": round(call_us, 3), "call_frac": frac(call_us),
        "call_us_graph": round(call_us_graph, 3), "call_frac_graph": frac(call_us_graph),
        "kernel_us_trace": k_us, "kernel_frac_trace": frac(k_us),
        "merge_us_trace": m_us,
        "traffic_bytes": traffic,
        "traffic_over_algorithmic": None if traffic is None else round(traffic / nbytes, 4),
        "target_frac": GATE_FRAC,
        "pass_call": frac(call_us) >= GATE_FRAC,
        "pass_kernel": None if k_us is None else frac(k_us) >= GATE_FRAC,
    }
    if cold_us_graph is not None:
        entry["call_us_cold_graph"] = round(cold_us_graph, 3)
        entry["call_frac_cold_graph"] = frac(cold_us_graph)
    if floors is not None:
        entry["floors"] = floors
        entry["floor_frac_read_one_launch"] = frac(floors["ring_bytes_read_one_launch_us"])
    return entry


CPU_REPS = 3  # oracle repetitions per timed part (about 10 s of CPU work on 16 threads)
COMPOSITE_VOCAB = 131072  # synthetic target vocabulary for the greedy acceptance step
COMPOSITE_MARGIN = 4096  # cache room for the tokens the composite keeps (a + 1 per iteration)


def composite(W, synth, D3, V4, full, tgt, cap, cap4, stream, ev, log, iters: int = 8,
              depths=(1, 2, 3, 4, 5)):
    """One speculative decode iteration at L = 1M, attention side only, for draft depths k and
    every acceptance a = 0..k: k draft steps (append + attend; windowed ring with k slack slots,
    or the contiguous cache), the target's append + verification of the k+1 candidates, greedy
    acceptance on synthetic logits, and the rollback of the k - a rejected tokens in the draft
    cache and the target cache. The draft tokens are built from the logits' argmax so that
    exactly a of them are accepted (checked on the device after the timed iterations), so each
    (k, a) iteration does its own accept and rollback work. Per-token cost = iteration cost /
    (a + 1) tokens. Also the no-speculation decode step (the target appends one token and attends
    everything)."""
    import numpy as np
    import torch

    dev = full.k.device
    dt = full.k.dtype
    Hq, Hkv, d, S, Wn = D3.n_q_heads, D3.n_kv_heads, D3.head_dim, D3.sink, D3.window
    Hq4, Hkv4, d4 = V4.n_q_heads, V4.n_kv_heads, V4.head_dim
    kmax = max(depths)
    n0 = int(full.seq_len.item())
    n4 = int(tgt.seq_len.item())
    # a ring with kmax slack slots holding the same sequence as the contiguous draft cache
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, dt, dev, slack=kmax)
    for p0, p1 in ((0, min(S, n0)), (max(S, n0 - Wn - kmax), n0)):
        ring.seq_len.fill_(p0)
        W.wmtp_ring_append(ring, full.k[0, :, p0:p1].permute(1, 0, 2).contiguous()[None],
                           full.v[0, :, p0:p1].permute(1, 0, 2).contiguous()[None], p1 - p0)
    scale3, scale4 = 1.0 / math.sqrt(d), 1.0 / math.sqrt(d4)
    tok_k = synth.token_rows(D3.seed + 1, synth.KNEW_ID, 0, 0, kmax, Hkv, d, dt, dev)
    tok_v = synth.token_rows(D3.seed + 1, synth.VNEW_ID, 0, 0, kmax, Hkv, d, dt, dev)
    cand_k = synth.token_rows(V4.seed + 1, synth.KNEW_ID, 0, 0, kmax + 1, Hkv4, d4, dt, dev)
    cand_v = synth.token_rows(V4.seed + 1, synth.VNEW_ID, 0, 0, kmax + 1, Hkv4, d4, dt, dev)
    q3 = synth.queries(D3.seed + 1, 0, 1, 1, Hq, d, dt, dev)
    q4 = synth.queries(V4.seed + 1, 0, 1, kmax + 1, Hq4, d4, dt, dev)
    out3 = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse3 = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
    out4 = torch.empty((1, kmax + 1, Hq4, d4), dtype=torch.float32, device=dev)
    lse4 = torch.empty((1, kmax + 1, Hq4), dtype=torch.float32, device=dev)
    ws_win = W.workspace(1, Hq, Hkv, d, 1, ring.capacity, dev)
    ws_full = W.workspace(1, Hq, Hkv, d, 1, cap, dev)
    V = COMPOSITE_VOCAB
    g = torch.Generator(device="cpu").manual_seed(D3.seed)
    logits_host = torch.randn((1, kmax + 1, V), generator=g).to(dt)
    logits = logits_host.to(dev)
    # the target's greedy choice per row (first maximum), from the same bf16 values
    pick = np.argmax(logits_host.float().numpy()[0], axis=1)
    choice = torch.empty((1, kmax + 1), dtype=torch.int32, device=dev)
    n_acc, nxt, n_drop = (torch.empty((1,), dtype=torch.int32, device=dev) for _ in range(3))
    res = {"vocab": V, "depths": list(depths), "windowed_iter_us": {}, "full_iter_us": {},
           "reduction": {}, "per_token_us": {}, "accepted_checked": True}

    def drafts_for(k, a):
        """k draft tokens of which exactly the first a equal the target's choices."""
        dr = [int(pick[i]) for i in range(a)]
        if a < k:
            dr.append(int((pick[a] + 1) % V))
        dr += [int(pick[i]) for i in range(len(dr), k)]
        return torch.tensor([dr], dtype=torch.int32, device=dev)

    def iteration(form, k, a):
        ws_acc = W.accept_workspace(1, k, V, dev)
        ws_ver = W.workspace(1, Hq4, Hkv4, d4, k + 1, cap4, dev)
        lg = logits[:, :k + 1].contiguous()
        dr = drafts_for(k, a)
        ch = choice[:, :k + 1].contiguous()
        qk = q4[:, :k + 1].contiguous()  # made once here, not a copy inside the timed iteration
        cache = ring if form == "windowed" else full

        def run():
            for i in range(k):
                if form == "windowed":
                    W.wmtp_draft_step_windowed(ring, tok_k[i:i + 1][None], tok_v[i:i + 1][None],
                                               q3, Hq, scale3, out3, lse3, ws_win)
                else:
                    W.wmtp_draft_step_full(full, tok_k[i:i + 1][None], tok_v[i:i + 1][None], q3,
                                           Hq, scale3, cap, out3, lse3, ws_full)
            W.wmtp_verify_step(tgt, cand_k[:k + 1][None], cand_v[:k + 1][None], qk, k + 1, Hq4,
                               scale4, cap4, out4[:, :k + 1], lse4[:, :k + 1], ws_ver)
            W.wmtp_greedy_accept(lg, k, dr, ch, n_acc, nxt, n_drop, ws_acc)
            W.wmtp_ring_rollback(cache, n_drop)
            W.wmtp_ring_rollback(tgt, n_drop)
        return run

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        marks = [ev() for _ in range(iters + 1)]
        marks[0].record(stream)
        for i in range(iters):
            fn()
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        us = sorted(1000.0 * marks[i].elapsed_time(marks[i + 1]) for i in range(iters))
        return us[len(us) // 2]

    for k in depths:
        tw, tf = [], []
        for a in range(k + 1):
            tw.append(timed(iteration("windowed", k, a)))
            ok = int(n_acc.item()) == a
            tf.append(timed(iteration("full", k, a)))
            ok = ok and int(n_acc.item()) == a
            res["accepted_checked"] = res["accepted_checked"] and ok
        res["windowed_iter_us"][str(k)] = [round(x, 1) for x in tw]
        res["full_iter_us"][str(k)] = [round(x, 1) for x in tf]
        res["reduction"][str(k)] = [round(1.0 - w / f, 4) for w, f in zip(tw, tf)]
        res["per_token_us"][str(k)] = {
            "windowed": [round(tw[a] / (a + 1), 1) for a in range(k + 1)],
            "full": [round(tf[a] / (a + 1), 1) for a in range(k + 1)]}
        log(f"composite k={k}: windowed {[round(x) for x in tw]} us, full {[round(x) for x in tf]} us "
            f"per iteration for a = 0..{k}")
    # every iteration rolls back what it did not accept, so the caches only grow by the accepted
    # tokens (draft cache) and accepted + 1 (target)
    assert int(full.seq_len.item()) >= n0 and int(tgt.seq_len.item()) >= n4
    one_k = cand_k[:1][None]
    one_v = cand_v[:1][None]
    one = torch.ones((1,), dtype=torch.int32, device=dev)
    ws1 = W.workspace(1, Hq4, Hkv4, d4, 1, cap4, dev)
    q1 = q4[:, :1].contiguous()

    def nospec():
        W.wmtp_verify_step(tgt, one_k, one_v, q1, 1, Hq4, scale4, cap4, out4[:, :1], lse4[:, :1],
                           ws1)
        W.wmtp_ring_rollback(tgt, one)  # keep the cache length fixed across repetitions
    res["no_speculation_step_us"] = round(timed(nospec), 1)
    res["note"] = ("attention-side cost of one decode iteration (eager launches) for draft depth k "
                   "and exactly a accepted drafts (lists indexed by a = 0..k; the drafts are built "
                   "from the synthetic logits' argmax and the device's acceptance count is checked: "
                   "accepted_checked); tokens per iteration = a + 1; per_token_us = iteration / "
                   "(a + 1); no_speculation_step_us includes a rollback of the token it appends")
    return res


def oracle_time(fn, reps: int = 3) -> float:
    """Mean wall time (us) of `reps` calls of an oracle function on the host."""
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    return (time.perf_counter() - t0) / reps * 1e6


def other_workloads(W, synth, configs, stream, ev, log, calls: int = 100, cpu: bool = False):
    """Draft steps of the tiny workload (L = 4096, fp32, 8q/2kv, d64, S4, W256), the mid-context
    workload (L = 131072, 32q/4kv, d128, S4, W2048) and the batched ring workload (8 ragged
    sequences, 16q/2kv, d128, S4, W2048):
      * attention-only calls, graph-replayed back to back (*_attn_us_graph);
      * for the mid-context and batched workloads also the fused step (append + attend, then a
        rollback of the token, so every call sees the same lengths): cold (each call after a
        cache flush, events around it; p50/p10/p90 of `calls`) and warm (graph-replayed);
      * with cpu=True, the float64 oracle on the same bytes (oracle_us, host cores).
    """
    import numpy as np
    import torch

    oracle = None
    if cpu:
        import oracle as oracle_mod
        oracle = oracle_mod
    dev = torch.device("cuda:0")
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    res = {}

    def time_calls(fn, cold):
        """cold: each call after a 512 MiB flush, events around the call (the flush keeps the GPU
        busy while the host queues the call, so the events bracket GPU work); p50/p10/p90.
        warm: `calls` calls captured in one HIP graph and replayed (back to back, no host launch
        gaps); mean."""
        if not cold:
            return {"mean": round(graph_us(fn, calls, reps=1), 2)}
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(calls):
            W.wmtp_llc_flush(flush_buf)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = sorted(1000.0 * a.elapsed_time(b) for a, b in pairs)
        return {"p50": round(us[len(us) // 2], 2), "p10": round(us[len(us) // 10], 2),
                "p90": round(us[(9 * len(us)) // 10], 2)}

    # ---- tiny draft step (fp32)
    T = configs.TINY
    L, Hq, Hkv, d, S, Wn = T.context, T.n_q_heads, T.n_kv_heads, T.head_dim, T.sink, T.window
    f32 = torch.float32
    n = L + 1
    full = W.KVCache.contiguous(1, Hkv, d, n, f32, dev)
    full.k[0] = synth.sequence_rows(T.seed, synth.K_ID, 0, 0, n, Hkv, d, f32, dev)
    full.v[0] = synth.sequence_rows(T.seed, synth.V_ID, 0, 0, n, Hkv, d, f32, dev)
    full.seq_len.fill_(n)
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, f32, dev)
    W.wmtp_ring_append(ring, full.k[0].permute(1, 0, 2).contiguous()[None],
                       full.v[0].permute(1, 0, 2).contiguous()[None], n)
    q = synth.queries(T.seed, 0, 1, 1, Hq, d, f32, dev)
    out = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    ws_f = W.workspace(1, Hq, Hkv, d, 1, n, dev)
    ws_w = W.workspace(1, Hq, Hkv, d, 1, ring.capacity, dev)
    res["tiny"] = {
        "workload": T.name,
        "full_attn_us_graph": round(graph_us(lambda: W.wmtp_draft_attn_full(
            full, q, Hq, scale, n, out, lse, ws_f), calls), 3),
        "windowed_attn_us_graph": round(graph_us(lambda: W.wmtp_draft_attn_windowed(
            ring, q, Hq, scale, out, lse, ws_w), calls), 3)}
    if cpu:
        kv = oracle.contiguous_kv(synth.host_array(full.k), synth.host_array(full.v), oracle.F32)
        qh = synth.host_array(q)
        res["tiny"]["oracle_us"] = {
            "full_attn": round(oracle_time(lambda: oracle.draft_full(qh, oracle.F32, kv, [n], scale)), 1),
            "windowed_attn": round(oracle_time(lambda: oracle.draft_windowed(
                qh, oracle.F32, kv, [n], S, Wn, scale)), 1)}
    del full, ring

    # ---- mid-context draft step
    M = configs.MID
    dt = torch.bfloat16
    L, Hq, Hkv, d, S, Wn = M.context, M.n_q_heads, M.n_kv_heads, M.head_dim, M.sink, M.window
    cap = L + 16
    full = W.KVCache.contiguous(1, Hkv, d, cap, dt, dev)
    for c0 in range(0, L, 1 << 16):
        c1 = min(L, c0 + (1 << 16))
        full.k[0, :, c0:c1] = synth.sequence_rows(M.seed, synth.K_ID, 0, c0, c1, Hkv, d, dt, dev,
                                                  M.k_scale)
        full.v[0, :, c0:c1] = synth.sequence_rows(M.seed, synth.V_ID, 0, c0, c1, Hkv, d, dt, dev)
    full.seq_len.fill_(L)
    ring = W.KVCache.ring(1, Hkv, d, S, Wn, dt, dev, slack=1)
    for p0, p1 in ((0, S), (L - Wn - 1, L)):
        ring.seq_len.fill_(p0)
        W.wmtp_ring_append(ring, full.k[0, :, p0:p1].permute(1, 0, 2).contiguous()[None],
                           full.v[0, :, p0:p1].permute(1, 0, 2).contiguous()[None], p1 - p0)
    kn = synth.token_rows(M.seed, synth.KNEW_ID, 0, L, L + 1, Hkv, d, dt, dev, M.k_scale)[None]
    vn = synth.token_rows(M.seed, synth.VNEW_ID, 0, L, L + 1, Hkv, d, dt, dev)[None]
    q = synth.queries(M.seed, 0, 1, 1, Hq, d, dt, dev)
    out = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
    one = torch.ones((1,), dtype=torch.int32, device=dev)
    ws_f = W.workspace(1, Hq, Hkv, d, 1, cap, dev)
    ws_w = W.workspace(1, Hq, Hkv, d, 1, ring.capacity, dev)
    scale = 1.0 / math.sqrt(d)

    def step_full():
        W.wmtp_draft_step_full(full, kn, vn, q, Hq, scale, cap, out, lse, ws_f)
        W.wmtp_ring_rollback(full, one)

    def step_win():
        W.wmtp_draft_step_windowed(ring, kn, vn, q, Hq, scale, out, lse, ws_w)
        W.wmtp_ring_rollback(ring, one)

    res["mid_context"] = {
        "workload": M.name,
        "full_attn_us_graph": round(graph_us(lambda: W.wmtp_draft_attn_full(
            full, q, Hq, scale, cap, out, lse, ws_f), 20), 3),
        "windowed_attn_us_graph": round(graph_us(lambda: W.wmtp_draft_attn_windowed(
            ring, q, Hq, scale, out, lse, ws_w), calls), 3),
        "full_step_us_cold": time_calls(step_full, True),
        "windowed_step_us_cold": time_calls(step_win, True),
        "full_step_us_warm": time_calls(step_full, False),
        "windowed_step_us_warm": time_calls(step_win, False),
        "note": "step = fused append + attend, then a rollback of the token (kernel ~3 us)"}
    if cpu:
        kv = oracle.contiguous_kv(synth.host_array(full.k[:, :, :L]),
                                  synth.host_array(full.v[:, :, :L]), oracle.BF16)
        qh = synth.host_array(q)
        res["mid_context"]["oracle_us"] = {
            "full_attn": round(oracle_time(lambda: oracle.draft_full(qh, oracle.BF16, kv, [L], scale)), 1),
            "windowed_attn": round(oracle_time(lambda: oracle.draft_windowed(
                qh, oracle.BF16, kv, [L], S, Wn, scale)), 1)}
        del kv
    log(f"mid-context: full {res['mid_context']['full_attn_us_graph']} us, windowed "
        f"{res['mid_context']['windowed_attn_us_graph']} us (attention, graph-replayed)")
    del full, ws_f

    # ---- batched ring draft step
    Bc = configs.BATCHED
    B, Hq, Hkv, d, S, Wn = Bc.batch, Bc.n_q_heads, Bc.n_kv_heads, Bc.head_dim, Bc.sink, Bc.window
    lens = [synth.uniform_int(Bc.seed, synth.LEN_ID, b, Bc.ragged_lo, Bc.context) for b in range(B)]
    ring = W.KVCache.ring(B, Hkv, d, S, Wn, dt, dev, slack=1)
    held = []  # host copies of what each ring holds: (positions, K rows, V rows)
    for b, n in enumerate(lens):  # the ring state after n appends: sinks and the last W + 1 tokens
        sub = W.KVCache(ring.k[b:b + 1], ring.v[b:b + 1], ring.pos[b:b + 1], ring.seq_len[b:b + 1],
                        1, Hkv, d, ring.capacity, S, Wn, ring.dtype)
        rows_k, rows_v = [], []
        for p0, p1 in ((0, S), (n - Wn - 1, n)):
            sub.seq_len.fill_(p0)
            rk = synth.token_rows(Bc.seed, synth.K_ID, b, p0, p1, Hkv, d, dt, dev)
            rv = synth.token_rows(Bc.seed, synth.V_ID, b, p0, p1, Hkv, d, dt, dev)
            W.wmtp_ring_append(sub, rk[None], rv[None], p1 - p0)
            rows_k.append(rk)
            rows_v.append(rv)
        if cpu:
            held.append((n, torch.cat(rows_k).permute(1, 0, 2).contiguous(),
                         torch.cat(rows_v).permute(1, 0, 2).contiguous()))
    kn = torch.stack([synth.token_rows(Bc.seed, synth.KNEW_ID, b, 0, 1, Hkv, d, dt, dev)
                      for b in range(B)])
    vn = torch.stack([synth.token_rows(Bc.seed, synth.VNEW_ID, b, 0, 1, Hkv, d, dt, dev)
                      for b in range(B)])
    q = synth.queries(Bc.seed, 0, B, 1, Hq, d, dt, dev)
    out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
    ones = torch.ones((B,), dtype=torch.int32, device=dev)
    ws_w = W.workspace(B, Hq, Hkv, d, 1, ring.capacity, dev)
    scale = 1.0 / math.sqrt(d)

    def step_batched():
        W.wmtp_draft_step_windowed(ring, kn, vn, q, Hq, scale, out, lse, ws_w)
        W.wmtp_ring_rollback(ring, ones)

    nbytes = 2 * B * (S + Wn) * Hkv * d * 2
    res["batched"] = {"workload": Bc.name,
                      "windowed_attn_us_graph": round(graph_us(lambda: W.wmtp_draft_attn_windowed(
                          ring, q, Hq, scale, out, lse, ws_w), calls), 3),
                      "windowed_step_us_warm": time_calls(step_batched, False),
                      "windowed_step_us_cold": time_calls(step_batched, True),
                      "attended_kv_bytes": nbytes,
                      "note": "step = fused append + attend for all 8 sequences, then a rollback"}
    if cpu:
        # the rings' rows with their logical positions: sinks, then the last W + 1 positions
        hk = np.stack([synth.host_array(k) for _, k, _ in held])
        hv = np.stack([synth.host_array(v) for _, _, v in held])
        segs = [[(0, 0, S), (n - Wn - 1, S, Wn + 1)] for n, _, _ in held]
        kv = oracle.LogicalKV(hk, hv, oracle.BF16, segs)
        qh = synth.host_array(q)
        res["batched"]["oracle_us"] = {"windowed_attn": round(oracle_time(
            lambda: oracle.draft_windowed(qh, oracle.BF16, kv, lens, S, Wn, scale)), 1)}
    log(f"batched: windowed attention {res['batched']['windowed_attn_us_graph']} us (graph-replayed)")
    return res


MASW_INTERVALS = (64, 8)  # raw tokens per memory slot


def masw_step(W, synth, D3, full, ring, Hq, scale, stream, ev, log, calls: int = 30):
    """MASW-style draft step at the million-token draft shapes: the ring's sinks + window plus
    one memory slot per r raw tokens (synthetic slot rows), for each r in MASW_INTERVALS.
    Median of back-to-back calls; algorithmic bytes = attended K/V rows + q + out."""
    import torch

    dev = full.k.device
    dt = full.k.dtype
    Hkv, d, S, Wn = D3.n_kv_heads, D3.head_dim, D3.sink, D3.window
    n = int(ring.seq_len.item())
    q = synth.queries(D3.seed + 2, 0, 1, 1, Hq, d, dt, dev)
    out = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
    res = {"context": n, "interval": [], "slots": [], "attn_us": [], "hbm_gbs": []}
    for r in MASW_INTERVALS:
        m = n // r
        slots = W.KVCache.contiguous(1, Hkv, d, m, dt, dev)
        for c0 in range(0, m, 1 << 16):  # synthetic slot rows, appended in pieces
            c1 = min(m, c0 + (1 << 16))
            W.wmtp_ring_append(slots, synth.token_rows(D3.seed + 3, 11, 0, c0, c1, Hkv, d, dt, dev)[None],
                               synth.token_rows(D3.seed + 3, 12, 0, c0, c1, Hkv, d, dt, dev)[None],
                               c1 - c0)
        ws = W.masw_workspace(1, Hq, Hkv, d, ring.capacity, m, dev)
        call = lambda: W.wmtp_draft_attn_masw(ring, slots, q, Hq, scale, m, out, lse, ws)
        call()
        marks = [ev() for _ in range(calls + 1)]
        torch.cuda.synchronize()
        marks[0].record(stream)
        for i in range(calls):
            call()
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        us = sorted(1000.0 * marks[i].elapsed_time(marks[i + 1]) for i in range(calls))[calls // 2]
        nbytes = 2 * (min(n, S + Wn) + m) * Hkv * d * 2 + Hq * d * 2 + Hq * (d + 1) * 4
        res["interval"].append(r)
        res["slots"].append(m)
        res["attn_us"].append(round(us, 2))
        res["hbm_gbs"].append(round(nbytes / (us * 1e-6) / 1e9, 1))
        log(f"masw r={r}: {m} slots, {us:.2f} us")
        del slots, ws
    return res


def read_probe(W, buf, out, stream, ev, reps: int = 5) -> float:
    """GB/s of one streaming read of the whole probe buffer (median of `reps` launches)."""
    times = []
    for _ in range(reps + 1):
        e0, e1 = ev(), ev()
        e0.record(stream)
        W.wmtp_probe_read(buf, out)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    t = sorted(times[1:])[reps // 2]
    return buf.numel() / (t * 1e-3) / 1e9


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def sweep(W, synth, D3, full, cap, Hq, scale, probe_buf, probe_out, stream, ev, log,
          calls: int = 100, warm_up: int = 20):
    """Single draft-step attention calls at the million-token draft shapes over a range of context
    lengths L (the step attends n = L + 1 tokens): windowed (ring holding sinks + window of the
    same sequence) and full (the first n rows of the contiguous cache), each timed per call with
    events after `warm_up` calls: cold (the caches flushed before every call) and warm (calls back
    to back behind a backlog read); median, p10 and p90 of `calls` calls. The one-call steps
    (append, then attend) of both forms are timed the same way."""
    import torch

    dev = full.k.device
    Hkv, d, S, Wn = D3.n_kv_heads, D3.head_dim, D3.sink, D3.window
    dt = full.k.dtype
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    q = synth.queries(D3.seed, 0, 1, 1, Hq, d, dt, dev)
    out = torch.empty((1, 1, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 1, Hq), dtype=torch.float32, device=dev)
    ws_full = W.workspace(1, Hq, Hkv, d, 1, cap, dev)
    ws_win = W.workspace(1, Hq, Hkv, d, 1, S + Wn, dev)
    res = {"L": [], "n": [], "windowed_slots": [], "full_us_cold": [], "windowed_us_cold": [],
           "full_us_warm": [], "windowed_us_warm": [], "full_step_us_cold": [],
           "windowed_step_us_cold": [], "full_step_us_warm": [], "windowed_step_us_warm": [],
           "full_gbs_cold": [], "windowed_gbs_cold": [], "full_over_windowed_cold": []}
    for L in SWEEP_L:
        n = L + 1
        if n + warm_up + 2 * calls > cap:
            raise ValueError("the contiguous cache has no room for the sweep's appended tokens")
        seq = torch.full((1,), n, dtype=torch.int32, device=dev)
        view = W.KVCache(full.k, full.v, None, seq, 1, Hkv, d, full.capacity, full.capacity, 0,
                         full.dtype)
        ring = W.KVCache.ring(1, Hkv, d, S, Wn, dt, dev)
        for p0, p1 in ((0, min(S, n)), (max(S, n - Wn), n)):
            if p1 <= p0:
                continue
            ring.seq_len.fill_(p0)
            kn = synth.token_rows(D3.seed, synth.K_ID, 0, p0, p1, Hkv, d, dt, dev)[None]
            vn = synth.token_rows(D3.seed, synth.V_ID, 0, p0, p1, Hkv, d, dt, dev)[None]
            W.wmtp_ring_append(ring, kn, vn, p1 - p0)
        slots = min(n, S + Wn)
        kn = synth.token_rows(D3.seed, synth.K_ID, 0, n, n + 1, Hkv, d, dt, dev)[None]
        vn = synth.token_rows(D3.seed, synth.V_ID, 0, n, n + 1, Hkv, d, dt, dev)[None]
        calls_of = {
            "full": lambda: W.wmtp_draft_attn_full(view, q, Hq, scale, cap, out, lse, ws_full),
            "windowed": lambda: W.wmtp_draft_attn_windowed(ring, q, Hq, scale, out, lse, ws_win),
            # the one-call steps (append, then attend; timing only): each call appends one more
            # token, so the full read grows by one key per call (at most 2 * calls + warm_up)
            "full_step": lambda: W.wmtp_draft_step_full(view, kn, vn, q, Hq, scale, cap, out, lse,
                                                        ws_full),
            "windowed_step": lambda: W.wmtp_draft_step_windowed(ring, kn, vn, q, Hq, scale, out,
                                                                lse, ws_win),
        }
        for name, call in calls_of.items():
            for _ in range(warm_up):
                call()
            cold, warm = [], []
            for _ in range(calls):
                e0, e1 = ev(), ev()
                W.wmtp_llc_flush(flush_buf)
                e0.record(stream)
                call()
                e1.record(stream)
                cold.append((e0, e1))
            W.wmtp_probe_read(probe_buf, probe_out, 1 << 30)  # backlog: the host runs ahead
            marks = [ev() for _ in range(calls + 1)]
            marks[0].record(stream)
            for i in range(calls):
                call()
                marks[i + 1].record(stream)
            torch.cuda.synchronize()
            cold_us = [1000.0 * a.elapsed_time(b) for a, b in cold]
            warm_us = [1000.0 * marks[i].elapsed_time(marks[i + 1]) for i in range(calls)]
            res[f"{name}_us_cold"].append({"p50": round(pct(cold_us, 0.5), 2),
                                           "p10": round(pct(cold_us, 0.1), 2),
                                           "p90": round(pct(cold_us, 0.9), 2)})
            res[f"{name}_us_warm"].append({"p50": round(pct(warm_us, 0.5), 2),
                                           "p10": round(pct(warm_us, 0.1), 2),
                                           "p90": round(pct(warm_us, 0.9), 2)})
        rows = {"full": n, "windowed": slots}
        for name in ("full", "windowed"):
            nbytes = 2 * rows[name] * Hkv * d * 2 + Hq * d * 2 + Hq * (d + 1) * 4
            t = res[f"{name}_us_cold"][-1]["p50"]
            res[f"{name}_gbs_cold"].append(round(nbytes / (t * 1e-6) / 1e9, 1))
        res["full_over_windowed_cold"].append(
            round(res["full_us_cold"][-1]["p50"] / res["windowed_us_cold"][-1]["p50"], 2))
        res["L"].append(L)
        res["n"].append(n)
        res["windowed_slots"].append(slots)
        log(f"sweep L={L}: full {res['full_us_cold'][-1]['p50']} us, windowed "
            f"{res['windowed_us_cold'][-1]['p50']} us (cold p50; steps "
            f"{res['full_step_us_cold'][-1]['p50']} / {res['windowed_step_us_cold'][-1]['p50']} us)")
        del ring
    return res


def cpu_baseline(full, tgt, ring, draft_q, ver_q, k, m, S, Wn, scale3, scale4, step_bytes, log,
                 other=None, gpu_calls=None):
    """The float64 oracle, as it stands, on the host cores: one full-context draft step, one
    windowed draft step and one verification over the same caches, scaled to a whole step; and,
    per workload, the oracle's time per attention call beside the GPU's (graph-replayed)."""
    import oracle
    from draft_attention_amd import configs, synth

    threads = oracle.max_threads()
    n3 = int(full.seq_len.item())
    n4 = int(tgt.seq_len.item())
    log(f"cpu baseline: copying caches to the host (n={n3}, {n4})")
    kv3 = oracle.contiguous_kv(synth.host_array(full.k[:, :, :n3]),
                               synth.host_array(full.v[:, :, :n3]), oracle.BF16)
    kv4 = oracle.contiguous_kv(synth.host_array(tgt.k[:, :, :n4]),
                               synth.host_array(tgt.v[:, :, :n4]), oracle.BF16)
    q3 = synth.host_array(draft_q[-1])
    q4 = synth.host_array(ver_q[-1])
    log(f"cpu baseline: oracle on {threads} threads")

    def timed(fn, reps):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t0) / reps

    reps = CPU_REPS
    t_full = timed(lambda: oracle.draft_full(q3, oracle.BF16, kv3, [n3], scale3), reps)
    t_win = timed(lambda: oracle.draft_windowed(q3, oracle.BF16, kv3, [n3], S, Wn, scale3), reps)
    t_ver = timed(lambda: oracle.verify(q4, oracle.BF16, kv4, [n4], scale4), reps)
    t_step = k * (t_full + t_win) + t_ver
    log(f"cpu baseline: full {t_full:.2f}s windowed {t_win * 1e3:.1f}ms verify {t_ver:.2f}s")
    per_config = {
        configs.MILLION.name: {
            "oracle_us": {"full_attn": round(t_full * 1e6, 1), "windowed_attn": round(t_win * 1e6, 1)},
            "gpu_us": None if gpu_calls is None else {"full_attn": round(gpu_calls["full"], 3),
                                                      "windowed_attn": round(gpu_calls["win"], 3)}},
        configs.VERIFY.name: {
            "oracle_us": {"verify_attn": round(t_ver * 1e6, 1)},
            "gpu_us": None if gpu_calls is None else {"verify_attn": round(gpu_calls["ver"], 3)}},
    }
    for key in ("tiny", "mid_context", "batched"):
        w = (other or {}).get(key)
        if not w or "oracle_us" not in w:
            continue
        gpu = {f"{form}_attn": w[f"{form}_attn_us_graph"] for form in ("full", "windowed")
               if f"{form}_attn_us_graph" in w}
        per_config[w["workload"]] = {"oracle_us": w["oracle_us"], "gpu_us": gpu}
    for v in per_config.values():
        if v["gpu_us"]:
            v["oracle_over_gpu"] = {c: round(v["oracle_us"][c] / v["gpu_us"][c], 1)
                                    for c in v["oracle_us"] if c in v["gpu_us"]}
    return {
        "value": round(step_bytes / t_step / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"one full-context draft step (32 heads x {n3} keys), one windowed draft step "
                   f"and one verification (4 x 32 heads x {n4} keys), each timed {reps} times "
                   f"(mean); whole step = 5 x (full + windowed) + verify = {t_step:.2f} s"),
        "draft_step_us": {"full_attn": round(t_full * 1e6, 1), "windowed_attn": round(t_win * 1e6, 1)},
        "verify_us": round(t_ver * 1e6, 1),
        "host": dict(host_cpu(), omp_threads=threads),
        "per_config": per_config,
        "per_config_note": "oracle_us: mean of 3 oracle calls per attention call (one draft step "
                           "or one verification) on the host cores; gpu_us: the same call "
                           "graph-replayed on the GPU",
    }


if __name__ == "__main__":
    main()
