#!/usr/bin/env python3
"""Benchmark of the verify step (spec_verify) on one MI355X.

Workload (default): B=64 requests, gamma=5 drafts each, vocabulary V=128256,
bf16 logits, temperature 1.0 (target logits 4 N(0,1) plus a Zipf-like bias,
draft logits = target + 0.5 N(0,1), drafts sampled from the draft distribution,
seeded uniforms).  One step = one spec_verify call over the whole batch: row
statistics of the 11 logit rows of every request, acceptance and first
rejection, residual / bonus sampling.  ``--mode greedy`` runs the same logits at
T = 0, ``--config N`` another workload (4: the ragged, mixed-temperature batch
through spec_verify_ex).

Inputs are resident in HBM before timing starts.  Steps rotate over C copies of
the logits totalling more than 1 GB, so that every call streams its logits
from HBM and not from the 256 MB last-level cache; C consecutive steps are
captured in one HIP graph and replayed.

Printed: one JSON line with the metric, the per-step time, the roofline figure
of the step (algorithmic bytes over the step's device time, from HIP events on
the launch stream around the timed region), the row-statistics kernel's own
time, the streaming-read ceiling, and the single-threaded CPU oracle's rate on
the same workloads (pinned to one core).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/s + achieved HBM GB/s vs peak (B×(2γ+1)×V logits)"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
PROFILE_PMC = os.path.join(PROFILES, "step_B64_g5_V128256_bf16.pmc.json")
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verification_spec_amd", "csrc", "specverify.hip")
PROBE_LIB = os.path.join(ROOT, "rejection_sampling_verification_spec_amd", "libsvprobe.so")
# the step's kernels on these workloads (every row has at most 512 sub-chunks, so the decision kernel
# also draws and k3_select is not launched)
STEP_KERNELS = ("k1_row_stats", "k2_decide_mass")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the kernel source with comments and blank space removed, so that
    stored counters stay valid across edits that change no code."""
    import re
    text = open(KERNEL_SRC, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
    text = re.sub(r"//[^\n]*", " ", text)                 # line comments
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0: enough for 1.2 GB)")
    ap.add_argument("--config", type=int, default=3, help="workload timed as the step, by its index in workloads.make_config (default 3: B = 64, gamma = 5, V = 128256 bf16)")
    ap.add_argument("--mode", choices=["stochastic", "greedy"], default="stochastic",
                    help="the B = 64, gamma = 5, V = 128256 bf16 batch at T = 1 or at T = 0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only (no sampler, filter, tree, other workloads, cold latency, probe)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU oracle time budget over all workloads")
    ap.add_argument("--eager", action="store_true", help="launch every step eagerly instead of graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarise rocprofv3 CSV output under DIR into profiles/")
    return ap.parse_args()


# --------------------------------------------------------------------------- profile summaries
_BENCH = "python3 bench.py"
PROFILE_COMMANDS = {
    "kt": f"rocprofv3 --kernel-trace --stats -d DIR/kt -o kt --output-format csv -- {_BENCH} "
          "--no-extras --no-cpu-baseline",
    "kt_greedy": f"rocprofv3 --kernel-trace --stats -d DIR/kt_greedy -o kt --output-format csv -- {_BENCH} "
                 "--mode greedy --no-extras --no-cpu-baseline",
    "kt_config4": f"rocprofv3 --kernel-trace --stats -d DIR/kt_config4 -o kt --output-format csv -- {_BENCH} "
                  "--config 4 --no-extras --no-cpu-baseline",
    "kt_extras": f"rocprofv3 --kernel-trace --stats -d DIR/kt_extras -o kt --output-format csv -- {_BENCH} "
                 "--no-cpu-baseline",
    "pmc_FETCH_SIZE": f"rocprofv3 --pmc FETCH_SIZE -d DIR/pmc_FETCH_SIZE -o pmc --output-format csv -- {_BENCH} "
                      "--steps 14 --warmup 7 --no-cpu-baseline --eager --no-extras",
    "pmc_WRITE_SIZE": f"rocprofv3 --pmc WRITE_SIZE -d DIR/pmc_WRITE_SIZE -o pmc --output-format csv -- {_BENCH} "
                      "--steps 14 --warmup 7 --no-cpu-baseline --eager --no-extras",
    "copy_FETCH_SIZE": f"rocprofv3 --pmc FETCH_SIZE -d DIR/copy_FETCH_SIZE -o pmc --output-format csv -- {_BENCH} "
                       "--copy-calibration",
    "copy_WRITE_SIZE": f"rocprofv3 --pmc WRITE_SIZE -d DIR/copy_WRITE_SIZE -o pmc --output-format csv -- {_BENCH} "
                       "--copy-calibration",
}
TRACE_TITLES = {
    "kt": "Kernel durations: the timed step, B=64, gamma=5, V=128256 bf16, T=1 (stochastic)",
    "kt_greedy": "Kernel durations: the timed step, B=64, gamma=5, V=128256 bf16, T=0 (greedy)",
    "kt_config4": "Kernel durations: the timed step, B=128, ragged gamma_b in 1..7, V=152064 bf16, "
                  "per-request T in {0, 0.6, 1} (spec_verify_ex)",
    "kt_extras": "Kernel durations: the default benchmark run (timed step plus the sampler, filtered, tree and "
                 "other-workload measurements)",
}
TRACE_FILES = {"kt": "kernels_B64_g5_V128256_bf16_T1.md", "kt_greedy": "kernels_B64_g5_V128256_bf16_greedy.md",
               "kt_config4": "kernels_B128_ragged_V152064_bf16_mixedT.md", "kt_extras": "kernels_benchmark_extras.md"}


def _kernel_short(name: str) -> str:
    """Kernel name with its template arguments spelled out (element type, request kind, filtering)."""
    import re
    m = re.search(r"::(k\w+)<([^>]*)>", name)
    if not m:
        m2 = re.search(r"\b(k_\w+|k\d\w*)\b", name)
        return m2.group(1) if m2 else name.split("(")[0][:60]
    kname, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    tags = [{"0": "f32", "1": "bf16"}.get(args[0], args[0])]
    if kname == "k1_row_stats" and len(args) == 3:
        tags.append({"0": "per-request T", "1": "stochastic", "2": "greedy"}.get(args[2], args[2]))
    elif kname == "k_tree_walk" and len(args) == 2:
        tags.append("own statistics" if args[1] == "true" else "statistics from K1")
    elif len(args) in (2, 3) and args[1] in ("true", "false"):
        tags.append("filtered" if args[1] == "true" else "plain")
        if len(args) == 3 and args[2] == "true":
            tags.append("draws")
    return f"{kname}<{', '.join(tags)}>"


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _bench_line(d):
    """The JSON line bench.py printed under the profiler (saved next to the trace as bench.json)."""
    p = os.path.join(d, "bench.json")
    if os.path.exists(p):
        for line in open(p):
            line = line.strip()
            if line.startswith("{"):
                return json.loads(line)
    return None


def summarize_profile(root: str):
    import csv
    import statistics
    os.makedirs(PROFILES, exist_ok=True)
    traces = {}
    for key, title in TRACE_TITLES.items():
        d = os.path.join(root, key)
        if not os.path.isdir(d):
            continue
        stats = list(csv.DictReader(open(_find_csv(d, "kernel_stats.csv"))))
        bl = _bench_line(d)
        lines = [f"# {title}", "", "Command (from the repository root, output under DIR):", "",
                 "    " + PROFILE_COMMANDS[key] + " > DIR/" + key + "/bench.json", "",
                 "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
                 "|---|---|---|---|---|---|"]
        avg = {}
        for r in stats:
            n = _kernel_short(r["Name"])
            avg[n] = float(r["AverageNs"]) / 1e3
            lines.append(f"| {n} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        if bl is not None:
            lines += ["", f"The same run's benchmark line: {bl['ms_per_step'] * 1e3:.2f} us per step on the host "
                          f"clock, {bl['extra']['device_us_per_step']:.2f} us per step between the HIP events "
                          f"({bl['config']['workload']}); step roofline fraction {bl['roofline']['frac']:.4f} "
                          f"({bl['roofline']['achieved']:.0f} GB/s of algorithmic bytes)."]
            # the timed step's own kernels (one instantiation of each): their averages summed
            k1_tag = {"kt": "stochastic", "kt_greedy": "greedy", "kt_config4": "per-request T"}.get(key)
            if k1_tag is not None:
                want = [f"k1_row_stats<bf16, {k1_tag}>",
                        "k2_decide_mass<bf16, plain>" if key == "kt_greedy" else "k2_decide_mass<bf16, plain, draws>"]
                if all(k in avg for k in want):
                    step_sum = sum(avg[k] for k in want)
                    bytes_step = bl["roofline"]["bytes_per_step"]
                    lines += ["", f"The step's kernels ({' + '.join(want)}) average {step_sum:.2f} us together: "
                                  f"{bytes_step / step_sum / 1e3:.0f} GB/s of the step's algorithmic bytes, fraction "
                                  f"{bytes_step / step_sum / 1e3 / HBM_PEAK_GBS:.4f} of 8 TB/s.  The event time per "
                                  "step also holds the gaps between the graph's kernel nodes (wider under the "
                                  "profiler)."]
        lines += ["", "The copy kernels are the benchmark's set-up (input copies), outside the timed region.", ""]
        open(os.path.join(PROFILES, TRACE_FILES[key]), "w").write("\n".join(lines))
        traces[key] = {"kernel_avg_us": avg, "bench": None if bl is None else
                       {"ms_per_step": bl["ms_per_step"], "device_us_per_step": bl["extra"]["device_us_per_step"],
                        "frac": bl["roofline"]["frac"]}}

    def pmc_medians(d):
        rows = list(csv.DictReader(open(_find_csv(os.path.join(root, d), "counter_collection.csv"))))
        by = {}
        for r in rows:
            by.setdefault(_kernel_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in by.items()}, {k: len(v) for k, v in by.items()}

    rec = {"kernel_source_sha256_16": source_hash(), "traces": traces}
    if os.path.isdir(os.path.join(root, "pmc_FETCH_SIZE")):
        fetch, nf = pmc_medians("pmc_FETCH_SIZE")
        write, _ = pmc_medians("pmc_WRITE_SIZE")
        cfetch, _ = pmc_medians("copy_FETCH_SIZE")
        cwrite, _ = pmc_medians("copy_WRITE_SIZE")
        copy_name = max(cfetch, key=lambda k: cfetch[k])   # the 1 GiB copy kernel (the fill reads nothing)
        copy_kib = (1 << 30) / 1024
        f_fetch, f_write = copy_kib / cfetch[copy_name], copy_kib / cwrite[copy_name]
        # the timed step's own instantiations: the stochastic row-statistics kernel (the per-request-T
        # one in the same run belongs to the separate row-statistics timing) and the plain K2
        step = [k for k in fetch if k.split("<")[0] in STEP_KERNELS
                and ("stochastic" in k if k.startswith("k1_") else "plain" in k)]
        per = {k: round((fetch[k] * f_fetch + write.get(k, 0.0) * f_write) * 1024) for k in step}
        step_bytes = sum(per.values())
        bytes_alg = 64 * 11 * 128256 * 2
        rec.update({"mode": "stochastic", "copy_kernel": copy_name, "copy_fetch_kib": cfetch[copy_name],
                    "copy_write_kib": cwrite[copy_name], "fetch_scale": f_fetch, "write_scale": f_write,
                    "fetch_kib_per_dispatch": {k: fetch[k] for k in step},
                    "write_kib_per_dispatch": {k: write.get(k) for k in step},
                    "hbm_bytes_per_launch": per, "hbm_bytes_per_step": step_bytes, "bytes_alg_per_step": bytes_alg,
                    "traffic_over_alg": step_bytes / bytes_alg,
                    "commands": {k: PROFILE_COMMANDS[k] for k in ("pmc_FETCH_SIZE", "pmc_WRITE_SIZE",
                                                                   "copy_FETCH_SIZE", "copy_WRITE_SIZE")}})
        lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE, KiB)", "",
                 "Workload: B=64, gamma=5, V=128256 bf16, T=1 (stochastic), eager launches.", "",
                 "Commands (from the repository root, output under DIR):", ""]
        lines += ["    " + PROFILE_COMMANDS[k] for k in ("pmc_FETCH_SIZE", "pmc_WRITE_SIZE", "copy_FETCH_SIZE",
                                                           "copy_WRITE_SIZE")]
        lines += ["", "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | bytes (scaled) |",
                  "|---|---|---|---|---|"]
        for k in fetch:
            b = (fetch[k] * f_fetch + write.get(k, 0.0) * f_write) * 1024
            lines.append(f"| {k} | {nf[k]} | {fetch[k]:.1f} | {write.get(k, float('nan')):.1f} | {b / 1e6:.2f} MB |")
        lines += ["", f"Calibration: the plain 1 GiB device copy ({copy_name}) reads {cfetch[copy_name]:.1f} KiB "
                  f"and writes {cwrite[copy_name]:.1f} KiB by these counters, so FETCH_SIZE is scaled by "
                  f"{f_fetch:.4f} and WRITE_SIZE by {f_write:.4f} to give bytes.", "",
                  f"The step (k1_row_stats + k2_decide_mass): {step_bytes / 1e6:.2f} MB per step against "
                  f"{bytes_alg / 1e6:.2f} MB algorithmic (ratio {step_bytes / bytes_alg:.4f}); the excess is "
                  f"the residual pass re-reading the sampled row pair of each request (and one sub-chunk of "
                  f"it for the draw).", ""]
        open(os.path.join(PROFILES, "hbm_traffic_B64_g5_V128256_bf16.md"), "w").write("\n".join(lines))
    json.dump(rec, open(PROFILE_PMC, "w"), indent=2)
    print(json.dumps(rec, indent=2))


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}), flush=True)


# --------------------------------------------------------------------------- timing helpers
def graph_time(torch, stream, one, copies, reps_target):
    """Per-call time of one(c) over the copies, captured in one graph and replayed."""
    with torch.cuda.stream(stream):
        one(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(copies):
            one(c)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, reps_target // copies)
    s0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - s0) / (reps * copies)


def verify_call(sv, w, t, tg, dr, cnt, out, ws, stream):
    """The step for workload w: spec_verify for a uniform batch, spec_verify_ex otherwise."""
    uniform = w.lens is None and w.scalar_temperature is not None
    greedy = uniform and w.scalar_temperature == 0.0

    def one(c):
        if uniform:
            sv.spec_verify(tg[c], None if greedy else dr[c], t["draft_tokens"], None if greedy else t["u_accept"],
                           t["u_sample"], float(w.scalar_temperature), accepted_count=cnt, out_tokens=out,
                           workspace=ws, stream=stream)
        else:
            sv.spec_verify_ex(tg[c], dr[c], t["draft_tokens"], t["u_accept"], t["u_sample"], t["temperature"],
                              t.get("lens"), accepted_count=cnt, out_tokens=out, workspace=ws, stream=stream)
    return one, ("spec_verify" if uniform else "spec_verify_ex")


def rotate(torch, t, elt, copies=None):
    cb = (t["target"].numel() + t["draft"].numel()) * elt
    if copies is None:
        copies = min(64, max(2, math.ceil(1.2e9 / cb)))
    return ([t["target"]] + [t["target"].clone() for _ in range(copies - 1)],
            [t["draft"]] + [t["draft"].clone() for _ in range(copies - 1)], copies, cb)


def time_config(sv, W, torch, cfg, greedy, dev, stream, cache, reps_target=100):
    """Throughput of one of the other workloads (inputs rotated over enough copies to exceed the
    last-level cache, at most 64: the smallest workloads run from cache, and say so)."""
    t0 = time.perf_counter()
    w = W.make_config(cfg, greedy=greedy)
    gen_s = time.perf_counter() - t0
    cache[(cfg, greedy)] = w
    t = w.to_torch(dev)
    elt = 2 if w.dtype == "bf16" else 4
    tg, dr, copies, cb = rotate(torch, t, elt)
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    ws = sv.new_workspace(sv.spec_verify_workspace_bytes(w.B, w.gamma, w.V, dt), dev)
    cnt = torch.empty(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.gamma + 1), dtype=torch.int32, device=dev)
    one, entry = verify_call(sv, w, t, tg, dr, cnt, out, ws, stream)
    with torch.cuda.stream(stream):
        one(0)
    torch.cuda.synchronize()
    rc, ro = cnt.cpu().clone(), out.cpu().clone()
    per = graph_time(torch, stream, one, copies, reps_target)
    assert torch.equal(cnt.cpu(), rc) and torch.equal(out.cpu(), ro), f"workload {cfg} replay differs"
    return {"workload": w.name, "entry": entry, "us_per_call": round(per * 1e6, 3),
            "positions_per_s": round(w.positions() / per, 1), "GBps_alg": round(w.bytes_alg() / per / 1e9, 1),
            "bytes_alg": w.bytes_alg(), "copies_rotated": copies, "cache_warm": copies * cb < 512e6,
            "alpha_hat": round(float(rc.float().sum()) / max(1, w.positions()), 4), "generate_s": round(gen_s, 1)}


def cold_latency(torch, np, one_call, stream, dev, n=41):
    """Per-call latency with the last-level cache flushed before each call (a 512 MB fill that the
    events exclude): median, p10 and p90 over n calls."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ts = []
    for k in range(n):
        with torch.cuda.stream(stream):
            flush.fill_(k & 0xff)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            one_call(k)
            b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    del flush
    q = np.percentile(np.array(ts), [10, 50, 90])
    return {"p10_us": round(float(q[0]), 2), "median_us": round(float(q[1]), 2), "p90_us": round(float(q[2]), 2),
            "calls": n}


def stream_probe(torch, dev, stream, nbytes, steps):
    """The streaming-read ceiling (libsvprobe): the same bytes per launch as the step's algorithmic
    bytes, rotated over copies beyond the last-level cache, 2816 workgroups as the row statistics."""
    lib = ctypes.CDLL(PROBE_LIB)
    lib.sv_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_stream_probe.restype = ctypes.c_int
    copies = max(2, math.ceil(1.2e9 / nbytes))
    bufs = [torch.full((nbytes,), k + 1, dtype=torch.uint8, device=dev) for k in range(copies)]
    groups = 2816
    out = torch.empty(groups, dtype=torch.int32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    with torch.cuda.stream(stream):     # torch's events must have been recorded once to be read
        for a, b in evs:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    for k in range(steps + 5):
        ev = None
        if k >= 5:
            a, b = evs[k - 5]
            ev = (ctypes.c_void_p * 2)(a.cuda_event, b.cuda_event)
        rc = lib.sv_stream_probe(ctypes.c_void_p(bufs[k % copies].data_ptr()), nbytes, groups,
                                 ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream), ev)
        assert rc == 0, rc
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / steps * 1e3
    del bufs
    return {"us_per_launch": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
            "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
            "workgroups": groups, "copies_rotated": copies}


# --------------------------------------------------------------------------- CPU oracle leg
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


FLAG_NAMES = ("accept_band", "cdf_band", "zero_mass_fallback", "top_p_cut_band", "cdf_band_prob_units")


def cpu_leg(W, budget_s, cache, headline_key):
    """The single-threaded fp64 oracle, pinned to one core, on every workload: at least one full call
    each, repeated within the budget; the headline is the benchmark's own workload."""
    import numpy as np

    import oracle
    oracle.load()
    old = os.sched_getaffinity(0)
    core = max(old)
    os.sched_setaffinity(0, {core})
    try:
        keys = [(0, False), (1, False), (2, False), (3, False), (3, True), (4, False)]
        per = {}
        share = budget_s / len(keys)
        for key in keys:
            w = cache.get(key) or W.make_config(key[0], greedy=key[1])
            cache[key] = w
            tr = oracle.run_workload(w, trace=True)     # flags: not timed
            flags = tr.flags
            n, spent = 0, 0.0
            while n == 0 or spent < share:
                c0 = time.perf_counter()
                oracle.run_workload(w, trace=False)
                spent += time.perf_counter() - c0
                n += 1
            name = f"config{key[0]}" + ("_greedy" if key[1] else "")
            per[name] = {"workload": w.name, "s_per_call": round(spent / n, 4), "calls": n,
                         "positions_per_s": round(w.positions() * n / spent, 2),
                         "near_boundary": {"flagged": int((flags != 0).sum()),
                                           **{b: int(((flags >> i) & 1).sum()) for i, b in enumerate(FLAG_NAMES)}},
                         "alpha_hat": round(float(np.sum(tr.accepted_count)) / max(1, w.positions()), 4)}
    finally:
        os.sched_setaffinity(0, old)
    head = per[headline_key]
    return {"value": head["positions_per_s"], "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{head['calls']} full calls of {head['workload']} "
                      f"({head['s_per_call']:.3f} s each; single-threaded fp64 C, gcc -O2), pinned to core {core}; "
                      f"every workload timed the same way under per_config, about {budget_s:.0f} s in all",
            "cpu_model": cpu_model(), "pinned_core": core, "host_cpus": os.cpu_count(), "per_config": per}


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(requests are independent, so a multi-GPU run would shard the batch with no exchange).",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return

    import rejection_sampling_verification_spec_amd as sv
    from rejection_sampling_verification_spec_amd import workloads as W

    sv.load_library()
    dev = torch.device("cuda:0")
    greedy = args.mode == "greedy"
    if greedy and args.config != 3:
        print("--mode greedy applies to the B = 64, gamma = 5, V = 128256 bf16 batch (--config 3)", file=sys.stderr)
        sys.exit(2)
    cache = {}
    t0 = time.perf_counter()
    w = W.make_config(args.config, greedy=greedy)
    cache[(args.config, greedy)] = w
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s")
    B, gamma, V = w.B, w.gamma, w.V
    positions = w.positions()
    bytes_alg = w.bytes_alg()                       # rows the method must read x V x element size
    elt = w.elt_bytes()
    formula_bytes = B * (2 * gamma + 1) * V * elt   # the metric's B x (2 gamma + 1) x V logits
    t = w.to_torch(dev)
    targets, drafts, copies, copy_bytes = rotate(torch, t, elt, args.copies or None)
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    count = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    need = sv.spec_verify_workspace_bytes(B, gamma, V, dt)
    ws = sv.new_workspace(need, dev)
    stream = torch.cuda.Stream()
    log(f"[bench] {copies} input copies ({copies * copy_bytes / 1e9:.2f} GB), workspace {need} B")
    one, entry = verify_call(sv, w, t, targets, drafts, count, out, ws, stream)

    with torch.cuda.stream(stream):
        one(0)
    torch.cuda.synchronize()
    ref_count, ref_out = count.cpu().clone(), out.cpu().clone()

    # HIP graphs: one graph holds `copies` consecutive steps (copy 0, 1, ..., C-1); a
    # shorter graph covers a remainder so that exactly K steps are timed
    graphs = {}

    def chain_graph(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(n):
                one(c)
        return g

    if not args.eager:
        graphs[copies] = chain_graph(copies)
        torch.cuda.synchronize()
        graphs[copies].replay()
        torch.cuda.synchronize()
        assert torch.equal(count.cpu(), ref_count) and torch.equal(out.cpu(), ref_out), "graph replay differs"

    def run_steps(n):
        with torch.cuda.stream(stream):
            if args.eager:
                for k in range(n):
                    one(k % copies)
                return
            full, rem = divmod(n, copies)
            for _ in range(full):
                graphs[copies].replay()
            if rem:
                if rem not in graphs:
                    graphs[rem] = chain_graph(rem)
                graphs[rem].replay()

    run_steps(args.warmup)
    if args.steps % copies and not args.eager and (args.steps % copies) not in graphs:
        graphs[args.steps % copies] = chain_graph(args.steps % copies)   # built before timing
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record(stream)
    run_steps(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    dev_s_per_step = e0.elapsed_time(e1) / 1e3 / args.steps
    host_ms = (h1 - h0) * 1e3
    ms_per_step = host_ms / args.steps
    value = positions * args.steps / (host_ms / 1e3)
    # every copy holds the same logits, so the last replay must reproduce the eager result
    assert torch.equal(count.cpu(), ref_count) and torch.equal(out.cpu(), ref_out), "timed replay differs"
    log(f"[bench] timed {args.steps} steps: host {host_ms:.3f} ms, device {dev_s_per_step * 1e3 * args.steps:.3f} ms")

    # the step's roofline: algorithmic bytes over the device time per step (HIP events on the
    # launch stream around the timed region)
    achieved = bytes_alg / dev_s_per_step / 1e9
    pmc = json.load(open(PROFILE_PMC)) if os.path.exists(PROFILE_PMC) else {}
    pmc_current = pmc.get("kernel_source_sha256_16") == source_hash()
    traffic = None
    if pmc_current and args.config == 3 and not greedy and pmc.get("mode") == "stochastic":
        traffic = pmc.get("hbm_bytes_per_step")
    kernels = STEP_KERNELS
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "scope": "whole step: " + " + ".join(kernels) + ("" if greedy else " (which also draws)"),
                "step_us": round(dev_s_per_step * 1e6, 3),
                "bytes_per_step": bytes_alg}

    # the row-statistics kernel on its own: event pairs the library records around its dispatch, on a
    # second pass over the same rotation through spec_verify_dbg, which runs the kernels spec_verify runs
    # (the instantiation of the timed steps); K1 reads every algorithmic byte once
    if args.config == 3:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        with torch.cuda.stream(stream):
            for a, b in evs:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        T0 = float(w.scalar_temperature)
        tg = None if greedy else t["u_accept"]
        with torch.cuda.stream(stream):
            for k, (a, b) in enumerate(evs):
                c = (args.warmup + k) % copies
                sv.spec_verify(targets[c], None if greedy else drafts[c], t["draft_tokens"], tg, t["u_sample"],
                               T0, accepted_count=count, out_tokens=out, workspace=ws, stream=stream,
                               k1_events=(a, b))
        torch.cuda.synchronize()
        k1_ms = [a.elapsed_time(b) for a, b in evs]
        k1_us = float(np.mean(k1_ms)) * 1e3
        roofline["k1_row_stats"] = {"instantiation": ("greedy" if greedy else "stochastic")
                                                     + " (the timed steps' own, through spec_verify_dbg)",
                                    "avg_us": round(k1_us, 3), "median_us": round(float(np.median(k1_ms)) * 1e3, 3),
                                    "min_us": round(min(k1_ms) * 1e3, 3),
                                    "max_us": round(max(k1_ms) * 1e3, 3),
                                    "achieved_GBps": round(bytes_alg / k1_us / 1e3, 1),
                                    "frac": round(bytes_alg / k1_us / 1e3 / HBM_PEAK_GBS, 4)}
    key = {(3, False): "kt", (3, True): "kt_greedy", (4, False): "kt_config4"}.get((args.config, greedy))
    tr = pmc.get("traces", {}).get(key) if pmc_current else None
    if tr:
        roofline["kernel_trace_avg_us"] = {k: round(v, 3) for k, v in tr["kernel_avg_us"].items()
                                           if k.split("<")[0] in STEP_KERNELS}

    extras = {}
    if not args.no_extras:
        extras["stream_probe"] = stream_probe(torch, dev, stream, bytes_alg, 50)
        log(f"[bench] stream probe {extras['stream_probe']}")

    # draft-side sampling (one token per row of softmax(z/T)) on the same draft logits:
    # B rows (one drafting step of the batch) and B*gamma rows (all positions)
    if not args.no_extras and args.config == 3 and not greedy:
        sample = {}
        for R in (B, B * gamma):
            rows = [d.view(B * gamma, V)[:R] for d in drafts]
            us = t["u_accept"].reshape(-1)[:R].contiguous()
            toks = torch.empty(R, dtype=torch.int32, device=dev)
            sws = sv.new_workspace(sv.spec_sample_workspace_bytes(R, V, sv.SV_BF16), dev)
            per = graph_time(torch, stream, lambda c, rows=rows, us=us, toks=toks, sws=sws:
                             sv.spec_sample(rows[c], us, 1.0, tokens=toks, workspace=sws, stream=stream),
                             copies, args.steps)
            sample[f"rows_{R}"] = {"us_per_call": round(per * 1e6, 3), "rows_per_s": round(R / per, 1),
                                   "GBps": round(R * V * 2 / per / 1e9, 1)}
        extras["spec_sample"] = sample
        log(f"[bench] spec_sample {sample}")

        # top-k / top-p filtered verification on the same logits at T = 0.7 (the pages' vLLM
        # example: temperature 0.7, top_p 0.9), with and without top_k = 50
        filtered = {}
        temps07 = torch.full((B,), 0.7, dtype=torch.float32, device=dev)
        fws = sv.new_workspace(sv.spec_verify_filtered_workspace_bytes(B, gamma, V, sv.SV_BF16), dev)
        for label, k, p in (("top_p0.9", None, 0.9), ("top_k50_top_p0.9", 50, 0.9)):
            tk = None if k is None else torch.full((B,), k, dtype=torch.int32, device=dev)
            tp = torch.full((B,), p, dtype=torch.float32, device=dev)

            def fstep(c, tk=tk, tp=tp):
                sv.spec_verify_filtered(targets[c], drafts[c], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                        temps07, None, top_k=tk, top_p=tp, accepted_count=count,
                                        out_tokens=out, workspace=fws, stream=stream)

            with torch.cuda.stream(stream):
                fstep(0)
            torch.cuda.synchronize()
            fc, fo = count.cpu().clone(), out.cpu().clone()
            per = graph_time(torch, stream, fstep, copies, args.steps)
            assert torch.equal(count.cpu(), fc) and torch.equal(out.cpu(), fo), "filtered replay differs"
            filtered[label] = {"us_per_call": round(per * 1e6, 3), "positions_per_s": round(positions / per, 1),
                               "alpha_hat": round(float(fc.float().mean()) / gamma, 4)}
        extras["spec_verify_filtered"] = filtered
        log(f"[bench] spec_verify_filtered {filtered}")

        # tree verification: 8 trees of width 4 and depth 3 (84 nodes) over the same vocabulary, T = 0.7
        t0 = time.perf_counter()
        tw = W.build_tree("B8_w4_d3_V128256_bf16_T0.7", 3000, 8, 4, 3, V, "bf16", target_scale=4.0, zipf=True,
                          sigma=0.5, temps=0.7)
        log(f"[bench] generated {tw.name} in {time.perf_counter() - t0:.1f}s")
        tt = tw.to_torch(dev)
        ttg, tdr, tcopies, _ = rotate(torch, tt, 2)
        tws = sv.new_workspace(sv.spec_verify_tree_workspace_bytes(tw.B, tw.N, V, sv.SV_BF16), dev)
        tc = torch.empty(tw.B, dtype=torch.int32, device=dev)
        to = torch.empty((tw.B, tw.N + 1), dtype=torch.int32, device=dev)
        tn = torch.empty((tw.B, tw.N), dtype=torch.int32, device=dev)

        def tstep(c):
            sv.spec_verify_tree(ttg[c], tdr[c], tt["parent"], tt["tokens"], tt["u_accept"], tt["u_sample"],
                                tt["temperature"], accepted_count=tc, out_tokens=to, out_nodes=tn, workspace=tws,
                                stream=stream)

        with torch.cuda.stream(stream):
            tstep(0)
        torch.cuda.synchronize()
        rc, ro, rn = tc.cpu().clone(), to.cpu().clone(), tn.cpu().clone()
        per = graph_time(torch, stream, tstep, tcopies, args.steps // 4)
        assert torch.equal(tc.cpu(), rc) and torch.equal(to.cpu(), ro), "tree replay differs"
        emitted = float(rc.sum()) + tw.B
        extras["spec_verify_tree"] = {
            "workload": tw.name, "us_per_call": round(per * 1e6, 3), "nodes_per_s": round(tw.B * tw.N / per, 1),
            "emitted_tokens_per_s": round(emitted / per, 1), "mean_accepted_path": round(float(rc.float().mean()), 3),
            # the walk reads the rows of the positions it visits (a wide tree's path is a small
            # share of its rows), so bandwidth is quoted on those bytes; every row of the trees
            # would be 'bytes_all_rows'
            "bytes_walked_rows": tw.bytes_walked(rn.numpy(), rc.numpy()),
            "GBps_walked_rows": round(tw.bytes_walked(rn.numpy(), rc.numpy()) / per / 1e9, 1),
            "bytes_all_rows": tw.bytes_alg()}
        log(f"[bench] spec_verify_tree {extras['spec_verify_tree']}")
        del ttg, tdr, tt

    if not args.no_extras:
        extras["cold_latency"] = cold_latency(torch, np, lambda k: one(k % copies), stream, dev)
        log(f"[bench] cold latency {extras['cold_latency']}")
        configs = {}
        for cfg, gr in [(0, False), (1, False), (2, False), (3, False), (3, True), (4, False)]:
            if (cfg, gr) == (args.config, greedy):
                continue
            name = f"config{cfg}" + ("_greedy" if gr else "")
            configs[name] = time_config(sv, W, torch, cfg, gr, dev, stream, cache)
            log(f"[bench] {name} {configs[name]}")
        extras["configs"] = configs

    cpu = None
    if not args.no_cpu_baseline:
        head = f"config{args.config}" + ("_greedy" if greedy else "")
        cpu = cpu_leg(W, args.cpu_seconds, cache, head)
        log(f"[bench] cpu baseline {cpu['value']} positions/s on {cpu['cpu_model']}")

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "entry": entry, "B": B, "gamma": gamma, "V": V, "input_dtype": w.dtype,
                   "temperature": "per request" if w.scalar_temperature is None else w.scalar_temperature,
                   "mode": args.mode, "copies_rotated": copies,
                   "launch": "eager" if args.eager else f"hip graph replay, {copies} steps per graph",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": {"device_us_per_step": round(dev_s_per_step * 1e6, 3),
                  "step_GBps_alg": round(bytes_alg / (ms_per_step / 1e3) / 1e9, 1),
                  "step_GBps_formula": round(formula_bytes / (ms_per_step / 1e3) / 1e9, 1),
                  "bytes_alg": bytes_alg, "bytes_formula": formula_bytes,
                  "alpha_hat": round(float(ref_count.float().sum()) / max(1, positions), 4),
                  **extras,
                  "kernel_source_sha256_16": source_hash()},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
