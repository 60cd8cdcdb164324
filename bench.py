"""Benchmark of the speculative-sampling verification step on one MI355X.

One step = one call of spec_verify_sample over a whole batch (row statistics, accept tests,
first-reject scan, residual mass, draw; greedy rows of the batch included), or of
spec_verify_greedy for a workload whose requests are all greedy (workload 2).  Inputs are
seeded synthetic workloads resident in HBM before timing; consecutive steps rotate over
enough input copies (> 2 x the 256 MB last-level cache) that no step reads cache-hot logits.

Prints one JSON line: verified positions/s (value) and logit GB/s with the HBM fraction from
an event-free timed region; per-kernel durations and the row statistics kernel's achieved
bandwidth from a second timed region of the same steps whose kernel dispatches record HIP
events; and the CPU oracle timed on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import subprocess
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20          # last-level (Infinity) cache
# launches of one call: row statistics, then accept tests + residual + draw (two-launch
# path), or the whole step (one-launch path: k_greedy1 for greedy calls, k_onepass else)
KERNELS = {"two": ["k_rowstats", "k_finish"], "one_greedy": ["k_greedy1"],
           "one": ["k_onepass"]}
PATHS = {"auto": 0, "two": 1, "one": 2}
DEFAULT_WORKLOAD = 5
WARMUP_SECONDS = 0.25
STEP_REPEATS = 9                # extra repeats of the K-step region, for the step time's spread
PROFILES = ROOT / "profiles"
COPY_BYTES = 1 << 30            # plain copy used to calibrate the HBM byte counters
KERNEL_SRC = ROOT / "speculative_sampling_verification_spec_amd" / "csrc" / "spec_verify.hip"


class HipEvents:
    """hipEvent_t handles through the HIP runtime (torch's events only see torch's own
    stream bookkeeping; these are recorded by the library on the stream it launches on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_digest() -> str:
    """sha256 of the kernel source's code: comments and whitespace removed, so that only a
    change of the code itself voids the committed counter runs."""
    import re
    text = KERNEL_SRC.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256(re.sub(r"\s+", "", text).encode()).hexdigest()


def traffic_for_current_kernel(kernel: str, workload: int):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter runs for this
    workload, or None if there are none or the kernel code changed since they were taken."""
    path = PROFILES / f"{kernel}_workload{workload}_traffic.json"
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if rec.get("code_sha256") != kernel_source_digest():
        return None
    return rec


def context_figures():
    """Context beside the 8 TB/s denominator, from the reference kernels of libspecbench.so on
    the current stream: the GPU time of one empty launch back to back, and the rate of a plain
    read stream (16-byte nontemporal loads) over 1 GiB buffers alternated beyond the
    last-level cache."""
    import torch
    L = ctypes.CDLL(str(ROOT / "speculative_sampling_verification_spec_amd" / "libspecbench.so"))
    L.spec_bench_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    L.spec_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        e0.record()
        for _ in range(reps):
            if fn() != 0:
                raise RuntimeError("reference kernel launch failed")
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    n = 2000
    timed(lambda: L.spec_bench_empty(200, stream), 2)
    empty_us = timed(lambda: L.spec_bench_empty(n, stream), 1) * 1e3 / n
    nbytes = COPY_BYTES
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    k = [0]

    def read():
        k[0] += 1
        return L.spec_bench_read(ctypes.c_void_p(bufs[k[0] % 3].data_ptr()), nbytes,
                                 ctypes.c_void_p(sink.data_ptr()), stream)

    timed(read, 6)
    ms = min(timed(read, 9) for _ in range(3))
    del bufs
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"empty_launch_us": round(empty_us, 2), "read_stream_GB_per_s": round(gbps, 1),
            "read_stream_frac": round(gbps / HBM_PEAK_GBPS, 4), "read_stream_bytes": nbytes}


def read_reference_us(nbytes: int) -> float:
    """GPU time of one plain read stream (libspecbench.so's 16-byte nontemporal reads, 64 KB per
    workgroup) over ``nbytes``, the reads rotating over enough buffers (> 2 x the last-level
    cache) that none is cache-hot: the minimum over three trials of the mean per read."""
    import torch
    L = ctypes.CDLL(str(ROOT / "speculative_sampling_verification_spec_amd" / "libspecbench.so"))
    L.spec_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = max(16, nbytes // 16 * 16)
    nbuf = max(3, math.ceil(2 * MALL_BYTES / nbytes) + 1)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    reps = max(nbuf, 30)

    def run(n):
        for i in range(n):
            if L.spec_bench_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nbytes,
                                 ctypes.c_void_p(sink.data_ptr()), stream) != 0:
                raise RuntimeError("reference read launch failed")

    run(reps)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        t0 = time.perf_counter()
        run(reps)
        torch.cuda.synchronize()
        best = min(best, (time.perf_counter() - t0) * 1e6 / reps)
    del bufs
    return best


def stop_row_bytes(w, nacc) -> int:
    """Bytes of the stop rows a call re-reads: two rows (target and draft) per sampled request
    that rejected a draft, one (the target's bonus row) per sampled request that accepted all."""
    es = 4 if w.dtype == "f32" else 2
    rows = sum(2 if int(nacc[b]) < int(w.gammas[b]) else 1
               for b in range(w.B) if w.temperatures[b] > 0)
    return rows * w.V * es


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, the reference the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE) are scaled by."""
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 5}), flush=True)


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_seconds: float, runs: int = 3):
    """The oracle, as it stands, on the benchmark workload, timed on this host's cores: the
    median of ``runs`` timed runs, each full passes over the first n requests (n sized so that
    all runs together take about ``target_seconds``)."""
    import oracle
    threads = oracle.max_threads()
    probe_n = min(w.B, 16)
    t = time.perf_counter()
    oracle.verify(w, requests=list(range(probe_n)), threads=threads)
    dt = time.perf_counter() - t
    per_run = target_seconds / runs
    n = int(min(w.B, max(probe_n, probe_n * per_run / max(dt, 1e-3))))
    reqs = list(range(n))
    rates, passes_done = [], []
    for _ in range(runs):
        passes = 0
        t = time.perf_counter()
        while True:
            oracle.verify(w, requests=reqs, threads=threads)
            passes += 1
            el = time.perf_counter() - t
            if el * (passes + 1) / passes > per_run or passes >= 100:
                break
        rates.append(int(w.gammas[:n].sum()) * passes / el)
        passes_done.append(passes)
    return {"value": float(np.median(rates)), "unit": "positions/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "runs_positions_per_s": [round(r, 1) for r in rates],
            "sample": f"median of {runs} runs, each {min(passes_done)}-{max(passes_done)} full "
                      f"pass(es) over the first {n} of {w.B} requests of the benchmark workload "
                      f"({int(w.gammas[:n].sum())} positions per pass, ~{per_run:.0f} s per run)"}


class Measured:
    """One workload measured on the GPU with the protocol below; holds its device inputs."""


def measure(sv, w, workload_id, args, path) -> Measured:
    """Warm-up, timed region A (step time, nothing on the stream but the library's kernels)
    and timed region B (per-kernel durations from events the kernels' dispatches record) for
    workload ``w``: every step is one call over the whole batch, rotating over enough input
    copies that no step reads cache-hot logits."""
    import torch
    m = Measured()
    m.w, m.workload_id = w, workload_id
    m.nbytes = w.compulsory_bytes
    copies = max(2, math.ceil(2 * MALL_BYTES / m.nbytes) + 1)
    m.copies = min(copies, max(2, (8 << 30) // max(m.nbytes, 1)))
    base = workloads_mod().to_torch(w)
    m.inputs = [base] + [dict(base, target=base["target"].clone(), draft=base["draft"].clone())
                         for _ in range(m.copies - 1)]
    m.code = sv.SPEC_F32 if w.dtype == "f32" else sv.SPEC_BF16
    m.ws = sv.alloc_workspace(w.B, w.gamma, w.V, m.code)
    m.out = torch.empty(w.R_t, dtype=torch.int32, device="cuda")
    m.nacc = torch.empty(w.B, dtype=torch.int32, device="cuda")
    hip = HipEvents()
    m.all_greedy = bool((w.temperatures == 0).all())  # the greedy entry point's workload
    inputs, out, nacc, ws, copies = m.inputs, m.out, m.nacc, m.ws, m.copies

    def step(k, probe):
        probe = probe if probe is not None or path == 0 else sv.make_probe(path=path)
        d = inputs[k % copies]
        if m.all_greedy:
            sv.spec_verify_greedy(d["target"], d["tokens"], w.gamma, out, nacc, ws,
                                  cu_draft=d["cu"], probe=probe)
        else:
            sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["uniforms"],
                                  d["temps"], w.gamma, out, nacc, ws, cu_draft=d["cu"],
                                  probe=probe)

    # Warm-up: the requested W steps, continued until at least 0.25 s of sustained load has
    # passed (the GPU's clocks settle some milliseconds into a run).
    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < WARMUP_SECONDS:
        step(warm, None)
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    m.warmup_steps_run = warm

    # Timed region A: the step time, with nothing on the stream but the library's kernels
    # (on this stack every recorded event leaves the GPU idle for several microseconds), and
    # each input copy's call marshalled once, as a serving loop would hold it.
    ctl = sv.make_probe(path=path) if path else None
    if m.all_greedy:
        calls = [sv.prepare_greedy(d["target"], d["tokens"], w.gamma, out, nacc, ws,
                                   cu_draft=d["cu"], probe=ctl) for d in inputs]
    else:
        calls = [sv.prepare_sample(d["target"], d["draft"], d["tokens"], d["uniforms"],
                                   d["temps"], w.gamma, out, nacc, ws, cu_draft=d["cu"], probe=ctl)
                 for d in inputs]
    t0 = time.perf_counter()
    for k in range(args.steps):
        calls[k % copies]()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.ms_per_step = (t1 - t0) * 1e3 / args.steps
    # The same region repeated (not part of the step time above): the spread of the per-step
    # time over repeats of K steps each.
    reps = []
    for _ in range(STEP_REPEATS):
        t0 = time.perf_counter()
        for k in range(args.steps):
            calls[k % copies]()
        torch.cuda.synchronize()
        reps.append((time.perf_counter() - t0) * 1e6 / args.steps)
    m.step_us_repeats = reps

    # Which launch path the calls took: the second launch's events are recorded only by
    # the two-launch path.
    evs = hip.create(4)
    step(0, sv.make_probe(events=evs, path=path))
    torch.cuda.synchronize()
    try:
        hip.elapsed_ms(evs[2], evs[3])
        m.taken = "two"
    except RuntimeError:
        hip.hip.hipGetLastError()
        m.taken = "one"
    hip.destroy(evs)
    m.kernels = KERNELS["one_greedy" if m.taken == "one" and m.all_greedy else m.taken]

    # Timed region B: the same steps again with per-kernel durations from events that each
    # kernel's dispatch records (probe events) on the stream it runs on.
    n_ev = 2 * len(m.kernels)
    evs = hip.create(n_ev * args.steps)
    probes = [sv.make_probe(events=evs[n_ev * k: n_ev * (k + 1)], path=path)
              for k in range(args.steps)]
    for k in range(args.steps):
        step(k, probes[k])
    torch.cuda.synchronize()
    m.per_kernel = {name: np.array([1e3 * hip.elapsed_ms(evs[n_ev * k + 2 * i],
                                                         evs[n_ev * k + 2 * i + 1])
                                    for k in range(args.steps)])
                    for i, name in enumerate(m.kernels)}
    hip.destroy(evs)
    m.per_kernel_us = {name: round(float(d.mean()), 2) for name, d in m.per_kernel.items()}
    m.step_kernels = sum(m.per_kernel.values())  # per step: the call's kernels back to back
    # the dominant kernel: the row-statistics stream, or the one launch that does everything
    m.rs_all = m.per_kernel[m.kernels[0]]
    m.rs_us = float(m.rs_all.mean())
    m.achieved = m.nbytes / (m.rs_us * 1e-6) / 1e9
    m.logit_gbps = m.nbytes / (m.ms_per_step * 1e-3) / 1e9
    # Last, after both timed regions (replaying a large graph slowed the kernels timed after
    # it): the same steps captured once in a HIP graph (enough of them for ~2 ms per replay, so
    # the events around a replay weigh little) and replayed, the GPU time per step without the
    # host's per-call cost, which bounds region A for the smallest workloads.
    m.graph_us_per_step = None
    if not args.no_graph:
        n_graph = copies * max(2, math.ceil(2000.0 / max(m.ms_per_step * 1e3, 1.0) / copies))
        m.graph_us_per_step = graph_us_per_call([(lambda k=k: step(k, None))
                                                 for k in range(n_graph)])
    m.stop_bytes = stop_row_bytes(w, m.nacc.cpu().numpy())
    return m


def read_floors(m: Measured) -> dict:
    """The plain read-stream reference at this workload's sizes, beside its step: the time to
    read its compulsory logit bytes once, and its stop rows once, and what two launches that
    did nothing but those two reads (plus one back-to-back launch) would reach."""
    t_logits = read_reference_us(m.nbytes)
    t_stop = read_reference_us(m.stop_bytes) if m.stop_bytes else 0.0
    t_launch = 1.3  # one empty launch back to back on this stack (context.empty_launch_us)
    floor = t_logits + t_stop + (t_launch if m.taken == "two" else 0.0)
    return {"read_logit_bytes_us": round(t_logits, 2), "stop_row_bytes": m.stop_bytes,
            "read_stop_row_bytes_us": round(t_stop, 2),
            "reads_only_frac": round(m.nbytes / (floor * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def finish_figures(m: Measured, floors: dict):
    """The finishing kernel against its own bytes: the stop rows it re-reads (overhead of the
    method, not in the metric's denominator) over its mean duration, beside the plain read
    stream's time for the same bytes.  None on the one-launch path."""
    us = m.per_kernel_us.get("k_finish")
    if us is None or not m.stop_bytes:
        return None
    gbps = m.stop_bytes / (us * 1e-6) / 1e9
    return {"kernel": "k_finish", "kernel_us": round(us, 2), "stop_row_bytes": m.stop_bytes,
            "GB_per_s": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "read_stop_row_bytes_us": floors["read_stop_row_bytes_us"]}


def rnd(x):
    return None if x is None else round(x, 2)


def pct(xs):
    return [round(float(np.percentile(xs, q)), 2) for q in (10, 50, 90)]


def workloads_mod():
    import workloads
    return workloads


def config_entry(m: Measured) -> dict:
    """A workload's figures for the per-config part of the line (same protocol as the main
    line; the 70%-of-peak bar is stated per call)."""
    w = m.w
    frac = m.logit_gbps / HBM_PEAK_GBPS
    floors = read_floors(m)
    return {"workload": f"{m.workload_id}: {w.name}", "B": w.B, "gamma_max": w.gamma, "V": w.V,
            "logit_dtype": w.dtype, "logit_bytes_per_step": m.nbytes,
            "entry_point": "spec_verify_greedy" if m.all_greedy else "spec_verify_sample",
            "launch_path": m.taken, "us_per_step": round(m.ms_per_step * 1e3, 2),
            "step_us_p10_p50_p90_over_repeats": pct(m.step_us_repeats),
            "graph_us_per_step": rnd(m.graph_us_per_step),
            "positions_per_s": round(w.positions / (m.ms_per_step * 1e-3), 1),
            "logit_GB_per_s": round(m.logit_gbps, 1), "hbm_frac": round(frac, 4),
            "meets_70pct_of_peak": bool(frac >= 0.70),
            "kernel_us": m.per_kernel_us,
            "dominant_kernel": m.kernels[0],
            "dominant_kernel_frac": round(m.achieved / HBM_PEAK_GBPS, 4),
            "k_finish_us": m.per_kernel_us.get("k_finish"),
            "dominant_kernel_traffic": (lambda r: None if r is None else r["hbm_bytes_per_launch"])(
                traffic_for_current_kernel(m.kernels[0], m.workload_id)),
            "step_kernel_us_p10_p50_p90": [round(float(np.percentile(m.step_kernels, q)), 1)
                                           for q in (10, 50, 90)],
            "read_reference": floors,
            "finish": finish_figures(m, floors)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD,
                    help="1..5; the JSON line is for workload 5 by default")
    ap.add_argument("--configs", default="1,2,3,4",
                    help="the other workloads measured in the same run with the same protocol "
                         "(comma list, or 'none'); reported under 'configs'")
    ap.add_argument("--config-entry", action="store_true",
                    help="print only this workload's entry of 'configs' (how the main run "
                         "measures each of them, in a process of its own)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing (profiling runs: the trace then ends with "
                         "timed region B)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain copy the byte counters are calibrated with")
    ap.add_argument("--path", choices=sorted(PATHS), default="auto",
                    help="launch path: the library's choice (auto), two launches, or one")
    ap.add_argument("--single-draft", type=int, default=0, metavar="B",
                    help="instead of a workload: a decode batch of B requests with one draft "
                         "each (V = 128256 bf16, T = 0.7)")
    ap.add_argument("--streams", type=int, default=1, metavar="S",
                    help="also time independent batches spread over S streams (context figure)")
    ap.add_argument("--shard", type=int, default=1, metavar="G",
                    help="instead of the JSON line: the workload split by requests over G GPUs "
                         "(ranges balanced by logit bytes), each GPU's share timed on this one "
                         "GPU in a process of its own; prints the shares and the slowest")
    ap.add_argument("--shard-index", type=int, default=-1, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this step has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); requests are independent, so several GPUs would each run "
              f"this step on their own share of the batch, with no communication",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    import speculative_sampling_verification_spec_amd as sv

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    t_gen = time.perf_counter()
    if args.single_draft > 0:
        B = args.single_draft
        w = workloads.generate(name=f"single-draft decode batch B={B} V=128256 bf16 T=0.7",
                               B=B, V=128256, dtype="bf16", gammas=[1] * B, dense=True,
                               target_sigma=3.0, draft_sigma=1.0, temperatures=0.7, seed=98)
        args.workload = 0
    else:
        w = workloads.config(args.workload)
    print(f"[bench] generated workload {args.workload} in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    if args.shard > 1 and args.shard_index < 0:
        print(json.dumps(time_shards(w, args)), flush=True)
        return
    if args.shard_index >= 0:  # a child of time_shards: this GPU's share of the requests
        lo, hi = workloads.shard_ranges(w, args.shard)[args.shard_index]
        w = w.requests(lo, hi)
    path = PATHS[args.path]
    m = measure(sv, w, args.workload, args, path)
    if args.config_entry:  # a child of the main run: this workload's figures only
        e = config_entry(m)
        if args.shard_index >= 0:  # the counters were taken on the whole workload
            e["dominant_kernel_traffic"] = None
        print(json.dumps(e), flush=True)
        return
    traffic = traffic_for_current_kernel(m.kernels[0], args.workload)
    value = w.positions / (m.ms_per_step * 1e-3)
    result = {
        "metric": "verified positions/sec and logit GB/s (fraction of HBM peak), 1 MI355X",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": m.warmup_steps_run,
        "ms_per_step": round(m.ms_per_step, 5),
        "step_us_p10_p50_p90_over_repeats": pct(m.step_us_repeats),
        "graph_us_per_step": rnd(m.graph_us_per_step),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {w.name}" if args.workload else w.name,
                   "B": w.B, "gamma_max": w.gamma,
                   "V": w.V, "logit_dtype": w.dtype, "positions_per_step": w.positions,
                   "logit_bytes_per_step": m.nbytes, "input_copies": m.copies,
                   "entry_point": "spec_verify_greedy" if m.all_greedy else "spec_verify_sample",
                   "launch_path": m.taken, "parallelism": "single GPU"},
        "logit_GB_per_s": round(m.logit_gbps, 1),
        "hbm_frac": round(m.logit_gbps / HBM_PEAK_GBPS, 4),
        "kernel_us": m.per_kernel_us,
        "step_kernel_us_p10_p50_p90": [round(float(np.percentile(m.step_kernels, q)), 1)
                                       for q in (10, 50, 90)],
        "roofline": {"bound": "hbm", "kernel": m.kernels[0], "kernel_us": round(m.rs_us, 2),
                     "kernel_us_p10_p50_p90": [round(float(np.percentile(m.rs_all, q)), 1)
                                               for q in (10, 50, 90)],
                     "achieved": round(m.achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(m.achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else traffic["hbm_bytes_per_launch"]},
        "cpu_baseline": None,
    }
    result["read_reference"] = read_floors(m)
    result["finish"] = finish_figures(m, result["read_reference"])
    result["commit"] = time_commit(sv, w, m.out, m.nacc, d=m.inputs[0], steps=args.steps)
    if args.streams > 1:
        result["independent_batches"] = time_streams(sv, w, m.inputs, m.code, path,
                                                      m.all_greedy, args.streams, args.steps)
    # The other workloads, each measured with the same protocol in a child process of its
    # own: inside one process, inputs allocated after another workload's streamed up to ~5%
    # slower (workload 4's k_rowstats 394 us after workload 5, 377 us first), so every
    # workload gets a process whose first allocations are its own.
    others = [] if args.configs == "none" or args.single_draft else \
        [int(c) for c in args.configs.split(",") if int(c) != args.workload]
    result["configs"] = {}
    for cid in others:
        cmd = [sys.executable, str(ROOT / "bench.py"), "--workload", str(cid), "--steps",
               str(args.steps), "--warmup", str(args.warmup), "--path", args.path,
               "--config-entry"] + (["--no-graph"] if args.no_graph else [])
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        sys.stderr.write(r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"measuring workload {cid} failed (exit {r.returncode})")
        result["configs"][str(cid)] = json.loads(r.stdout.strip().splitlines()[-1])
    result["context"] = context_figures()
    result["ngram"] = time_ngram(sv, steps=args.steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def time_shards(w, args) -> dict:
    """The workload split by requests over G GPUs: each share is the same call over fewer
    requests, with no communication, so each is timed alone on this GPU (a child process per
    share, the same protocol as the main line); a G-GPU step lasts as long as its slowest
    share."""
    import workloads
    G = args.shard
    shares = []
    for k, (lo, hi) in enumerate(workloads.shard_ranges(w, G)):
        cmd = [sys.executable, str(ROOT / "bench.py"), "--workload", str(args.workload),
               "--steps", str(args.steps), "--warmup", str(args.warmup), "--path", args.path,
               "--shard", str(G), "--shard-index", str(k), "--config-entry", "--no-graph"]
        print(f"[bench] share {k} of {G}: requests {lo}..{hi - 1}", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        sys.stderr.write(r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"measuring share {k} failed (exit {r.returncode})")
        e = json.loads(r.stdout.strip().splitlines()[-1])
        e["requests"] = [lo, hi]
        shares.append(e)
    slowest = max(s["us_per_step"] for s in shares)
    return {"workload": f"{args.workload}: {w.name}", "gpus_modelled": G,
            "split": "by requests, contiguous ranges balanced by logit bytes; no communication",
            "shares": shares, "step_us_slowest_share": slowest,
            "positions_per_s_all_gpus": round(w.positions / (slowest * 1e-6), 1),
            "logit_GB_per_s_all_gpus": round(w.compulsory_bytes / (slowest * 1e-6) / 1e9, 1)}


NGRAM = dict(B=512, capacity=8192, n_min=2, n_max=5, gamma=8, seed=77)


def time_streams(sv, w, inputs, code, path, all_greedy, nstreams, steps):
    """Calls over independent batches, round-robin over `nstreams` streams (default
    priority), each stream with its own workspace and outputs (calls on one stream run in
    order), so that one call's chain of dependent steps can overlap another's logit stream.  A
    context figure for serving loops that keep several batches in flight; the step time above
    is one call after another."""
    import torch
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    own = [(sv.alloc_workspace(w.B, w.gamma, w.V, code),
            torch.empty(w.R_t, dtype=torch.int32, device="cuda"),
            torch.empty(w.B, dtype=torch.int32, device="cuda")) for _ in range(nstreams)]
    ctl = sv.make_probe(path=path) if path else None
    calls = []
    for k in range(len(inputs) * nstreams):
        d, s = inputs[k % len(inputs)], streams[k % nstreams]
        ws, out, nacc = own[k % nstreams]
        if all_greedy:
            calls.append(sv.prepare_greedy(d["target"], d["tokens"], w.gamma, out, nacc, ws,
                                           cu_draft=d["cu"], probe=ctl, stream=s))
        else:
            calls.append(sv.prepare_sample(d["target"], d["draft"], d["tokens"], d["uniforms"],
                                           d["temps"], w.gamma, out, nacc, ws, cu_draft=d["cu"],
                                           probe=ctl, stream=s))
    torch.cuda.synchronize()
    n = max(steps, len(calls)) * nstreams
    for k in range(len(calls)):
        calls[k]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n):
        calls[k % len(calls)]()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / n
    return {"streams": nstreams, "calls": n, "us_per_call": round(us, 2),
            "positions_per_s": round(w.positions / (us * 1e-6), 1),
            "hbm_frac": round(w.compulsory_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def graph_us_per_call(calls, reps=5):
    """GPU time per call of ``calls`` (closures enqueueing one call each), captured once in a
    HIP graph and replayed: what a serving loop that captures its step pays, without the
    Python-side cost of eager calls."""
    import torch
    for c in calls[:2]:
        c()  # code objects load outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / len(calls))
    del g
    return best


def host_us_per_call(call, steps):
    """Wall time per eager call, back to back (the Python binding's cost included)."""
    import torch
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps


def time_ngram(sv, steps):
    """spec_ngram_propose (with the CSR packing) on self-repeating synthetic contexts: GPU time
    per call from graph replay over copies of the contexts that together exceed the last-level
    cache (so the contexts come from HBM, as after a verification step), the context bytes
    over that time, and the eager wall time per call."""
    import math
    import torch
    import workloads
    c = NGRAM
    seq, length = workloads.token_contexts(c["B"], c["capacity"], seed=c["seed"])
    B, g = c["B"], c["gamma"]
    copies = max(2, math.ceil(2 * (256 << 20) / seq.nbytes) + 1)
    seqs = [torch.from_numpy(seq).cuda() for _ in range(copies)]
    len_d = torch.from_numpy(length).cuda()
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    dense = torch.empty(B * g, dtype=torch.int32, device="cuda")
    cu = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    packed = torch.empty(B * g, dtype=torch.int32, device="cuda")

    def caller(sq):
        return lambda: sv.spec_ngram_propose(sq, len_d, c["n_min"], c["n_max"], g, counts,
                                             dense, cu, packed)

    gpu_us = graph_us_per_call([caller(sq) for sq in seqs])
    host_us = host_us_per_call(caller(seqs[0]), steps)
    nbytes = 4 * int(length.sum())
    return {"workload": f"B={B} contexts of up to {c['capacity']} tokens (mean {length.mean():.0f}), "
                        f"n {c['n_min']}..{c['n_max']}, gamma {g}",
            "gpu_us_per_call": round(gpu_us, 2), "context_GB_per_s": round(nbytes / gpu_us / 1e3, 1),
            "host_us_per_call": round(host_us, 2),
            "proposals_per_request": round(float(counts.float().mean()), 3)}


def time_commit(sv, w, out, nacc, d, steps):
    """spec_verify_commit on the last step's outputs, appending to histories with room for
    every call made here, and counting: GPU time per call from graph replay, and the eager
    wall time per call; not part of ``value`` (the step of the verification)."""
    import torch
    cap = (2 + 20 * 6 + steps + 8) * (w.gamma + 1)
    seq = torch.zeros((w.B, cap), dtype=torch.int32, device="cuda")
    ln = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    stats = torch.zeros(5, dtype=torch.int64, device="cuda")
    hist = torch.zeros(w.gamma + 1, dtype=torch.int64, device="cuda")
    call = lambda: sv.spec_verify_commit(out, nacc, w.gamma, seq, ln, cu_draft=d["cu"],
                                         stats=stats, accept_hist=hist)
    gpu_us = graph_us_per_call([call] * 20)
    host_us = host_us_per_call(call, steps)
    st = stats.cpu().numpy()
    return {"gpu_us_per_call": round(gpu_us, 2), "host_us_per_call": round(host_us, 2),
            "acceptance_rate": round(float(st[1] / max(st[0], 1)), 4),
            "tokens_per_pass": round(float(st[2] / max(st[3], 1)), 4)}


if __name__ == "__main__":
    main()
