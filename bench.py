#!/usr/bin/env python3
"""Benchmark of the verify step (spec_verify) on one MI355X.

Workload: B=64 requests, gamma=5 drafts each, vocabulary V=128256, bf16 logits,
temperature 1.0 (target logits 4 N(0,1) plus a Zipf-like bias, draft logits =
target + 0.5 N(0,1), drafts sampled from the draft distribution, seeded
uniforms).  One step = one spec_verify call over the whole batch: row
statistics of the 11 logit rows of every request, acceptance and first
rejection, residual / bonus sampling.

Inputs are resident in HBM before timing starts.  Steps rotate over C copies of
the logits totalling more than 1 GB, so that every call streams its logits
from HBM and not from the 256 MB last-level cache; C consecutive steps are
captured in one HIP graph and replayed.

Printed: one JSON line with the metric, the per-step time, the roofline figure
of the dominant kernel (row statistics, timed with HIP events that the library
records around it on the launch stream) and the single-threaded CPU oracle's
rate on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/s + achieved HBM GB/s vs peak (B×(2γ+1)×V logits)"
HBM_PEAK_GBS = 8000.0
PROFILE_PMC = os.path.join(ROOT, "profiles", "k1_row_stats_B64_g5_V128256_bf16.pmc.json")
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verification_spec_amd", "csrc", "specverify.hip")


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
    ap.add_argument("--mode", choices=["stochastic", "greedy"], default="stochastic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tree", action="store_true", help="skip the tree-verification measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations' timings and the cold-latency distribution")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    ap.add_argument("--eager", action="store_true", help="launch every step eagerly instead of graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarise rocprofv3 CSV output under DIR (kt/, pmc_FETCH_SIZE/, pmc_WRITE_SIZE/, "
                         "copy_FETCH_SIZE/, copy_WRITE_SIZE/) into profiles/")
    return ap.parse_args()


# --------------------------------------------------------------------------- profile summaries
PROFILE_COMMANDS = {
    "kt": "rocprofv3 --kernel-trace --stats -d DIR/kt -o kt --output-format csv -- python3 bench.py --no-configs",
    "pmc_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -d DIR/pmc_FETCH_SIZE -o pmc --output-format csv -- "
                      "python3 bench.py --steps 14 --warmup 7 --no-cpu-baseline --eager --no-configs",
    "pmc_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -d DIR/pmc_WRITE_SIZE -o pmc --output-format csv -- "
                      "python3 bench.py --steps 14 --warmup 7 --no-cpu-baseline --eager --no-configs",
    "copy_FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -d DIR/copy_FETCH_SIZE -o pmc --output-format csv -- "
                       "python3 bench.py --copy-calibration",
    "copy_WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -d DIR/copy_WRITE_SIZE -o pmc --output-format csv -- "
                       "python3 bench.py --copy-calibration",
}


def _kernel_short(name: str) -> str:
    """Kernel name with its template arguments spelled out (element type, request kind, filtering)."""
    import re
    m = re.search(r"::(k\w+)<([^>]*)>", name)
    if not m:
        return name.split("(")[0][:60]
    kname, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
    tags = [{"0": "f32", "1": "bf16"}.get(args[0], args[0])]
    if kname == "k1_row_stats" and len(args) == 3:
        tags.append({"0": "per-request T", "1": "stochastic", "2": "greedy"}.get(args[2], args[2]))
    elif len(args) == 2 and args[1] in ("true", "false"):
        tags.append("filtered" if args[1] == "true" else "plain")
    return f"{kname}<{', '.join(tags)}>"


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_profile(root: str):
    import csv
    import statistics
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    # kernel trace statistics
    stats = list(csv.DictReader(open(_find_csv(os.path.join(root, "kt"), "kernel_stats.csv"))))
    lines = ["# Kernel durations: B=64, gamma=5, V=128256 bf16, T=1 (stochastic)", "",
             "Command (from the repository root, output under DIR):", "",
             "    " + PROFILE_COMMANDS["kt"], "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    k1_avg_ns = None
    for r in stats:
        n = _kernel_short(r["Name"])
        lines.append(f"| {n} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        if n == "k1_row_stats<bf16, stochastic>":
            k1_avg_ns = float(r["AverageNs"])
    lines += ["", "Which call runs which kernels: the timed steps (spec_verify, T = 1) run "
              "k1_row_stats<bf16, stochastic>, k2_decide_mass<bf16, plain> and k3_select<bf16, plain>; "
              "the K1 timing pass (spec_verify_ex) runs k1_row_stats<bf16, per-request T>; the filtered "
              "measurement (spec_verify_filtered, T = 0.7, top_p = 0.9 with and without top_k = 50) runs "
              "k1_row_stats<bf16, per-request T>, k_filter_capture, k_filter_deep_count (with top_k = 50), "
              "k_filter_resolve, k_filter_general and the filtered k2 / k3; the tree measurement (spec_verify_tree, 8 trees of width 4 and depth 3) runs "
              "k1_row_stats<bf16, per-request T> and k_tree_walk; the draft-side sampling measurement runs "
              "k_sample_stats and k_sample_pick.  The copy kernels "
              "are the benchmark's set-up (input copies), outside the timed region.", ""]
    open(os.path.join(out_dir, "kernels_B64_g5_V128256_bf16.md"), "w").write("\n".join(lines))

    def pmc_medians(d):
        rows = list(csv.DictReader(open(_find_csv(os.path.join(root, d), "counter_collection.csv"))))
        by = {}
        for r in rows:
            by.setdefault(_kernel_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in by.items()}, {k: len(v) for k, v in by.items()}

    fetch, nf = pmc_medians("pmc_FETCH_SIZE")
    write, nw = pmc_medians("pmc_WRITE_SIZE")
    cfetch, _ = pmc_medians("copy_FETCH_SIZE")
    cwrite, _ = pmc_medians("copy_WRITE_SIZE")
    copy_name = max(cfetch, key=lambda k: cfetch[k])   # the 1 GiB copy kernel (the fill reads nothing)
    copy_kib = (1 << 30) / 1024
    f_fetch = copy_kib / cfetch[copy_name]
    f_write = copy_kib / cwrite[copy_name]
    K1 = "k1_row_stats<bf16, stochastic>"
    k1_bytes = (fetch[K1] * f_fetch + write[K1] * f_write) * 1024
    bytes_alg = 64 * 11 * 128256 * 2
    rec = {"kernel": "k1_row_stats", "mode": "stochastic", "kernel_source_sha256_16": source_hash(),
           "fetch_kib_per_dispatch": fetch[K1], "write_kib_per_dispatch": write[K1],
           "copy_kernel": copy_name, "copy_fetch_kib": cfetch[copy_name], "copy_write_kib": cwrite[copy_name],
           "fetch_scale": f_fetch, "write_scale": f_write, "hbm_bytes_per_launch": round(k1_bytes),
           "bytes_alg_per_launch": bytes_alg, "traffic_over_alg": k1_bytes / bytes_alg,
           "k1_avg_us_kernel_trace": None if k1_avg_ns is None else k1_avg_ns / 1e3,
           "commands": {k: PROFILE_COMMANDS[k] for k in ("pmc_FETCH_SIZE", "pmc_WRITE_SIZE", "copy_FETCH_SIZE",
                                                          "copy_WRITE_SIZE")}}
    json.dump(rec, open(PROFILE_PMC, "w"), indent=2)
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE, KiB)", "",
             "Workload: B=64, gamma=5, V=128256 bf16, T=1 (stochastic), eager launches.", "",
             "Commands (from the repository root, output under DIR):", ""]
    lines += ["    " + PROFILE_COMMANDS[k] for k in ("pmc_FETCH_SIZE", "pmc_WRITE_SIZE", "copy_FETCH_SIZE",
                                                       "copy_WRITE_SIZE")]
    lines += ["", "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |", "|---|---|---|---|"]
    for k in fetch:
        lines.append(f"| {k} | {nf[k]} | {fetch[k]:.1f} | {write.get(k, float('nan')):.1f} |")
    lines += ["", f"Calibration: the plain 1 GiB device copy ({copy_name}) reads {cfetch[copy_name]:.1f} KiB "
              f"and writes {cwrite[copy_name]:.1f} KiB by these counters, so FETCH_SIZE is scaled by "
              f"{f_fetch:.4f} and WRITE_SIZE by {f_write:.4f} to give bytes.",
              "", f"{K1}: {k1_bytes / 1e6:.2f} MB per launch against {bytes_alg / 1e6:.2f} MB algorithmic "
              f"(ratio {k1_bytes / bytes_alg:.4f}).", ""]
    open(os.path.join(out_dir, "hbm_traffic_B64_g5_V128256_bf16.md"), "w").write("\n".join(lines))
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


def time_config(sv, W, torch, math, cfg, greedy, dev, stream, reps_target=100):
    """Throughput of spec_verify (uniform T) or spec_verify_ex (per-request T and lengths) on one of
    the configurations, inputs rotated over enough copies to exceed the last-level cache where that
    fits in 1.2 GB (at most 64 copies: the smallest configurations run from cache, and say so)."""
    t0 = time.perf_counter()
    w = W.make_config(cfg, greedy=greedy)
    gen_s = time.perf_counter() - t0
    t = w.to_torch(dev)
    elt = 2 if w.dtype == "bf16" else 4
    copy_bytes = (t["target"].numel() + t["draft"].numel()) * elt
    copies = min(64, max(2, math.ceil(1.2e9 / copy_bytes)))
    tg = [t["target"]] + [t["target"].clone() for _ in range(copies - 1)]
    dr = [t["draft"]] + [t["draft"].clone() for _ in range(copies - 1)]
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    ws = sv.new_workspace(sv.spec_verify_workspace_bytes(w.B, w.gamma, w.V, dt), dev)
    cnt = torch.empty(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.gamma + 1), dtype=torch.int32, device=dev)
    uniform = w.lens is None and w.scalar_temperature is not None

    def one(c):
        if uniform:
            sv.spec_verify(tg[c], dr[c], t["draft_tokens"], t["u_accept"], t["u_sample"], float(w.scalar_temperature),
                           accepted_count=cnt, out_tokens=out, workspace=ws, stream=stream)
        else:
            sv.spec_verify_ex(tg[c], dr[c], t["draft_tokens"], t["u_accept"], t["u_sample"], t["temperature"],
                              t.get("lens"), accepted_count=cnt, out_tokens=out, workspace=ws, stream=stream)

    with torch.cuda.stream(stream):
        one(0)
    torch.cuda.synchronize()
    rc, ro = cnt.cpu().clone(), out.cpu().clone()
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
    per = (time.perf_counter() - s0) / (reps * copies)
    assert torch.equal(cnt.cpu(), rc) and torch.equal(out.cpu(), ro), f"config {cfg} replay differs"
    return {"workload": w.name, "entry": "spec_verify" if uniform else "spec_verify_ex",
            "us_per_call": round(per * 1e6, 3), "positions_per_s": round(w.positions() / per, 1),
            "GBps_alg": round(w.bytes_alg() / per / 1e9, 1), "bytes_alg": w.bytes_alg(),
            "copies_rotated": copies, "cache_warm": copies * copy_bytes < 512e6,
            "alpha_hat": round(float(rc.float().sum()) / max(1, w.positions()), 4),
            "generate_s": round(gen_s, 1)}


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

    lib = sv.load_library()
    dev = torch.device("cuda:0")
    greedy = args.mode == "greedy"
    t0 = time.perf_counter()
    w = W.make_config(3, greedy=greedy)
    log(f"[bench] generated {w.name} in {time.perf_counter() - t0:.1f}s")
    B, gamma, V = w.B, w.gamma, w.V
    T = float(w.scalar_temperature)
    positions = w.positions()
    bytes_alg = w.bytes_alg()                       # rows the method must read x V x 2 B
    formula_bytes = B * (2 * gamma + 1) * V * 2     # the metric's B x (2 gamma + 1) x V logits
    t = w.to_torch(dev)
    copy_bytes = (t["target"].numel() + t["draft"].numel()) * 2
    copies = args.copies or max(2, math.ceil(1.2e9 / copy_bytes))
    targets = [t["target"]] + [t["target"].clone() for _ in range(copies - 1)]
    drafts = [t["draft"]] + [t["draft"].clone() for _ in range(copies - 1)]
    count = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    need = sv.spec_verify_workspace_bytes(B, gamma, V, sv.SV_BF16)
    ws = sv.new_workspace(need, dev)
    stream = torch.cuda.Stream()
    log(f"[bench] {copies} input copies ({copies * copy_bytes / 1e9:.2f} GB), workspace {need} B")

    def step(c, s):
        return sv.spec_verify(targets[c], None if greedy else drafts[c], t["draft_tokens"],
                              None if greedy else t["u_accept"], t["u_sample"], T,
                              accepted_count=count, out_tokens=out, workspace=ws, stream=s)

    # eager reference result
    with torch.cuda.stream(stream):
        step(0, stream)
    torch.cuda.synchronize()
    ref_count, ref_out = count.cpu().clone(), out.cpu().clone()

    # HIP graphs: one graph holds `copies` consecutive steps (copy 0, 1, ..., C-1);
    # a shorter graph covers a remainder so that exactly K steps are timed
    graphs = {}

    def chain_graph(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(n):
                step(c, stream)
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
                    step(k % copies, stream)
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
    dev_ms = e0.elapsed_time(e1)
    host_ms = (h1 - h0) * 1e3
    ms_per_step = host_ms / args.steps
    value = positions * args.steps / (host_ms / 1e3)
    # every copy holds the same logits, so the last replay must reproduce the eager result
    assert torch.equal(count.cpu(), ref_count) and torch.equal(out.cpu(), ref_out), "timed replay differs"
    log(f"[bench] timed {args.steps} steps: host {host_ms:.3f} ms, device {dev_ms:.3f} ms")

    # dominant kernel: row statistics, timed by events the library records around it
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k, (a, b) in enumerate(evs):
            c = (args.warmup + k) % copies
            sv.spec_verify_ex(targets[c], drafts[c], t["draft_tokens"], t["u_accept"], t["u_sample"],
                              t["temperature"], None, accepted_count=count, out_tokens=out, workspace=ws,
                              stream=stream, k1_events=(a, b))
    torch.cuda.synchronize()
    k1_ms = [a.elapsed_time(b) for a, b in evs]
    k1_avg_s = float(np.mean(k1_ms)) / 1e3
    achieved = bytes_alg / k1_avg_s / 1e9
    traffic = None
    if os.path.exists(PROFILE_PMC):
        pmc = json.load(open(PROFILE_PMC))
        if pmc.get("kernel_source_sha256_16") == source_hash() and pmc.get("mode") == args.mode:
            traffic = pmc.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k1_row_stats", "kernel_avg_us": round(k1_avg_s * 1e6, 3),
                "bytes_per_launch": bytes_alg}

    # draft-side sampling (one token per row of softmax(z/T)) on the same draft logits:
    # 64 rows (one drafting step of the batch) and 320 rows (all five positions)
    sample = {}
    if not greedy:
        for R in (B, B * gamma):
            rows = [d.view(B * gamma, V)[:R] for d in drafts]
            us = t["u_accept"].reshape(-1)[:R].contiguous()
            toks = torch.empty(R, dtype=torch.int32, device=dev)
            sws = torch.empty(sv.spec_sample_workspace_bytes(R, V, sv.SV_BF16), dtype=torch.uint8, device=dev)

            def sstep(c, R=R, rows=rows, us=us, toks=toks, sws=sws):
                sv.spec_sample(rows[c], us, T, tokens=toks, workspace=sws, stream=stream)

            with torch.cuda.stream(stream):
                sstep(0)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for c in range(copies):
                    sstep(c)
            with torch.cuda.stream(stream):
                for _ in range(3):
                    g.replay()
            torch.cuda.synchronize()
            reps = max(1, args.steps // copies)
            s0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    g.replay()
            torch.cuda.synchronize()
            per = (time.perf_counter() - s0) / (reps * copies)
            sample[f"rows_{R}"] = {"us_per_call": round(per * 1e6, 3), "rows_per_s": round(R / per, 1),
                                   "GBps": round(R * V * 2 / per / 1e9, 1)}
        log(f"[bench] spec_sample {sample}")

    # top-k / top-p filtered verification on the same logits at T = 0.7 (the pages' vLLM
    # example: temperature 0.7, top_p 0.9), with and without top_k = 50
    filtered = {}
    if not greedy:
        temps07 = torch.full((B,), 0.7, dtype=torch.float32, device=dev)
        fws = torch.empty(sv.spec_verify_filtered_workspace_bytes(B, gamma, V, sv.SV_BF16), dtype=torch.uint8,
                          device=dev)
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
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for c in range(copies):
                    fstep(c)
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            reps = max(1, args.steps // copies)
            s0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    g.replay()
            torch.cuda.synchronize()
            per = (time.perf_counter() - s0) / (reps * copies)
            assert torch.equal(count.cpu(), fc) and torch.equal(out.cpu(), fo), "filtered replay differs"
            filtered[label] = {"us_per_call": round(per * 1e6, 3), "positions_per_s": round(positions / per, 1),
                               "alpha_hat": round(float(fc.float().mean()) / gamma, 4)}
        log(f"[bench] spec_verify_filtered {filtered}")

    # tree verification: 8 trees of width 4 and depth 3 (84 nodes) over the same vocabulary, T = 0.7
    tree = {}
    if not greedy and not args.no_tree:
        t0 = time.perf_counter()
        tw = W.build_tree("B8_w4_d3_V128256_bf16_T0.7", 3000, 8, 4, 3, V, "bf16", target_scale=4.0, zipf=True,
                          sigma=0.5, temps=0.7)
        log(f"[bench] generated {tw.name} in {time.perf_counter() - t0:.1f}s")
        tt = tw.to_torch(dev)
        tcopies = max(2, math.ceil(1.2e9 / ((tt["target"].numel() + tt["draft"].numel()) * 2)))
        ttg = [tt["target"]] + [tt["target"].clone() for _ in range(tcopies - 1)]
        tdr = [tt["draft"]] + [tt["draft"].clone() for _ in range(tcopies - 1)]
        tws = torch.empty(sv.spec_verify_tree_workspace_bytes(tw.B, tw.N, V, sv.SV_BF16), dtype=torch.uint8,
                          device=dev)
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
        rc, ro = tc.cpu().clone(), to.cpu().clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(tcopies):
                tstep(c)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // (4 * tcopies))
        s0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(reps):
                g.replay()
        torch.cuda.synchronize()
        per = (time.perf_counter() - s0) / (reps * tcopies)
        assert torch.equal(tc.cpu(), rc) and torch.equal(to.cpu(), ro), "tree replay differs"
        emitted = float(rc.sum()) + tw.B
        tree = {"workload": tw.name, "us_per_call": round(per * 1e6, 3), "nodes_per_s": round(tw.B * tw.N / per, 1),
                "emitted_tokens_per_s": round(emitted / per, 1), "mean_accepted_path": round(float(rc.float().mean()), 3),
                "GBps_alg": round(tw.bytes_alg() / per / 1e9, 1)}
        log(f"[bench] spec_verify_tree {tree}")

    # cold per-call latency of the timed call, and the other configurations' throughput
    latency, configs = None, {}
    if not args.no_configs:
        latency = cold_latency(torch, np, lambda k: step(k % copies, stream), stream, dev)
        log(f"[bench] cold latency {latency}")
        runs = [(0, False), (1, False), (2, False), (4, False)] + ([(3, True)] if not greedy else [])
        for cfg, gr in runs:
            key = f"config{cfg}" + ("_greedy" if gr else "")
            configs[key] = time_config(sv, W, torch, math, cfg, gr, dev, stream)
            log(f"[bench] {key} {configs[key]}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n, spent = 0, 0.0
        while spent < args.cpu_seconds or n == 0:
            c0 = time.perf_counter()
            oracle.run_workload(w, trace=False)
            spent += time.perf_counter() - c0
            n += 1
        cpu = {"value": round(positions * n / spent, 2), "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} full calls of the same B=64 workload (single-threaded fp64 C, gcc -O2), "
                         f"{spent:.1f} s", "host_cpus": os.cpu_count(), "host": platform.processor() or
                         platform.machine()}

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
        "config": {"workload": w.name, "B": B, "gamma": gamma, "V": V, "input_dtype": "bf16",
                   "temperature": T, "mode": args.mode, "copies_rotated": copies,
                   "launch": "eager" if args.eager else f"hip graph replay, {copies} steps per graph",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": {"step_GBps_alg": round(bytes_alg / (ms_per_step / 1e3) / 1e9, 1),
                  "step_GBps_formula": round(formula_bytes / (ms_per_step / 1e3) / 1e9, 1),
                  "bytes_alg": bytes_alg, "bytes_formula": formula_bytes,
                  "device_ms_per_step": round(dev_ms / args.steps, 5),
                  "k1_us_min": round(min(k1_ms) * 1e3, 3), "k1_us_max": round(max(k1_ms) * 1e3, 3),
                  "alpha_hat": round(float(ref_count.float().mean()) / gamma, 4),
                  "spec_sample": sample,
                  "spec_verify_filtered": filtered,
                  "spec_verify_tree": tree,
                  "cold_latency": latency,
                  "configs": configs,
                  "kernel_source_sha256_16": source_hash()},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
