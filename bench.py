#!/usr/bin/env python3
"""Benchmark of the all-gather matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--variant auto]

One step = one agmm_run (the whole hot path: gather/slot sync/tile schedule/
MFMA GEMM/epilogue, as the chosen variant does them) over one batch of seeded
synthetic inputs already resident in HBM.  Prints ONE JSON line.

value      : 2*m*k*n_local / (wall time per step), TFLOP/s, timed with events
             around exactly K steps (eager calls; launch-bound steps shorter
             than GRAPH_MAX_STEP_MS: one replay of a HIP graph holding the K
             steps).  Before the timed region: W warmup steps, then untimed
             steps for SETTLE_S of wall time (the clocks' ramp).
step_ms    : median / p10 / p90 of the K per-step times (eager: events
             between the steps; graph: per-step means of repeated replays).
roofline   : the dominant kernel (the MFMA GEMM, with its split-K reduction
             when it has one) timed per launch with HIP events on the stream
             it is launched on, against the MI355X dense bf16/fp16 MFMA peak
             (2.5 PFLOP/s), or against HBM (8 TB/s, algorithmic bytes) for
             workloads below the ridge point (the skinny one); next to it the
             same kernel's per-launch time from the committed rocprofv3 trace
             of this workload (profiles/kernel_trace_*.json).
workloads  : the skinny (8x16x4096->1792) and staged (8x1024x8192->3584)
             configurations measured the same way, so that their targets rest
             on this run too.
gather     : the gather copy alone (agmm_gather) on the same shards, GB/s of
             payload (m*k*elem) and of HBM traffic (read + write).
variants_ms: the same problem through the fused, staged and unfused paths.
cpu_baseline: the CPU oracle on a bounded sample of output rows, plus whole
             small workloads on one thread and on all of them.
At most one plan (two internal streams) is alive at any time, so that the
copy stream never shares a hardware queue with another plan's streams.
"""
from __future__ import annotations

import argparse
import faulthandler
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s of gather(A)@B (frac of bf16 MFMA peak) + gather GB/s, 1 MI355X"
PEAK_TFLOPS = {0: 2500.0, 1: 2500.0, 2: 157.3}   # bf16, fp16 dense MFMA; fp32 vector
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
GRAPH_MAX_STEP_MS = 0.25
# After the W warmup steps, untimed steps continue until this much wall time
# has passed: the GPU's clocks take more than ~10 ms of load to settle, and a
# short timed region would otherwise measure the ramp, not the kernels.
SETTLE_S = 0.2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--variant", default=None, help="auto|fused|staged|unfused|skinny")
    ap.add_argument("--also", default="2,3,4",
                    help="other workloads measured into the `workloads` field ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as K eager calls even when they are launch-bound")
    ap.add_argument("--only-run", action="store_true",
                    help="warmup + settle + K steps of the main path, then 3 gather copies of the "
                         "same shards (the known-size copy that calibrates HBM counters); for profilers")
    ap.add_argument("--no-settle", action="store_true",
                    help="--only-run without the untimed settle steps (counter runs: each dispatch "
                         "is slow under the profiler, and counters do not depend on the clock)")
    ap.add_argument("--launches-per-step", type=int, default=1,
                    help="--summarize-trace: dominant-kernel launches one step makes (staged: chunks)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the profiles/ summary of a rocprofv3 --kernel-trace --stats CSV run "
                         "of --only-run")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ traffic summary from rocprofv3 --pmc FETCH_SIZE and "
                         "--pmc WRITE_SIZE CSV runs of --only-run")
    ap.add_argument("--summarize-timeline", metavar="DIR",
                    help="write the profiles/ kernel timeline (copy / GEMM overlap) of a rocprofv3 "
                         "--kernel-trace CSV run of --only-run")
    ap.add_argument("--command", default="", help="profiler command line, recorded in summaries")
    return ap.parse_args()


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("gemm_mfma.hip", "skinny.hip", "gather_f32.hip", "agmm_kernels.h"):
        with open(os.path.join(ROOT, "all_gather_gemm_agmm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def resolve_variant(w, variant):
    variant = variant or w.variant
    if variant == "auto":
        variant = "skinny" if (w.m <= 256 and w.dtype != 2) else "fused"
    return variant


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    i = (len(xs) - 1) * q
    lo, hi = int(math.floor(i)), int(math.ceil(i))
    return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)


def traffic_from_profiles(workload_name: str, variant: str):
    """HBM bytes per launch of the dominant kernel, from committed rocprofv3
    PMC summaries; None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}_{variant}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def trace_from_profiles(workload_name: str, variant: str):
    """Per-launch time of the dominant kernel from the committed rocprofv3
    kernel trace of `bench.py --only-run` (None if absent or taken on other
    kernel sources)."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload_name}_{variant}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_sha") != kernel_source_sha():
        return None
    return d


# ------------------------------------------------------------ profile summaries
def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


MAIN_KERNELS = ("gemm_m16_kernel", "gemm_mfma_kernel", "skinny_splitk_kernel", "skinny_fullk_kernel",
                "gemm_f32_kernel")


def _short(name: str) -> str:
    for key in MAIN_KERNELS + ("splitk_reduce_kernel", "skinny_reduce_kernel", "gather_kernel",
                               "transpose16_kernel"):
        if key in name:
            return key
    return name[:48]


def summarize_trace(args, w, variant):
    """Kernel statistics of a `--only-run` trace, plus the per-launch times of
    the dominant kernel over the K timed steps alone (its last launches before
    the 3 calibration copies), which is what bench.py's roofline times."""
    rows = _csv_rows(args.summarize_trace, "kernel_stats.csv")
    name = f"kernel_trace_{w.name}_{variant}"
    lines = [f"# rocprofv3 kernel trace: {w.name}, {variant} path", "",
             f"command: `{args.command}`", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    out = []
    for r in rows:
        calls = int(r.get("Calls", 0) or 0)
        avg_ns = float(r.get("AverageNs", 0) or 0)
        out.append({"kernel": r.get("Name", ""), "calls": calls, "avg_us": avg_ns / 1e3,
                    "min_us": float(r.get("MinNs", 0) or 0) / 1e3,
                    "max_us": float(r.get("MaxNs", 0) or 0) / 1e3,
                    "pct": float(r.get("Percentage", 0) or 0)})
    for o in sorted(out, key=lambda o: -o["pct"]):
        lines.append(f"| {_short(o['kernel'])} | {o['calls']} | {o['avg_us']:.2f} | "
                     f"{o['min_us']:.2f} | {o['max_us']:.2f} | {o['pct']:.1f} |")
    # per-dispatch times of the timed steps
    disp = _csv_rows(args.summarize_trace, "kernel_trace.csv")
    disp.sort(key=lambda r: int(r["Start_Timestamp"]))
    main = next(k for k in MAIN_KERNELS if any(_short(r["Kernel_Name"]) == k for r in disp))
    mains = [r for r in disp if _short(r["Kernel_Name"]) == main]
    k_launches = args.steps * args.launches_per_step
    timed = mains[-k_launches:]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    # the step's companion kernels (split-K reduction, transposed copy of B),
    # one per dominant launch or one per step
    side = {}
    for key in ("splitk_reduce_kernel", "skinny_reduce_kernel", "transpose16_kernel"):
        n_side = args.steps if key == "transpose16_kernel" else k_launches
        rs = [r for r in disp if _short(r["Kernel_Name"]) == key][-n_side:]
        if rs:
            side[key] = sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs) / len(rs)
    summary = {"workload": w.name, "variant": variant, "kernel": main, "kernel_sha": kernel_source_sha(),
               "timed_launches": len(durs), "avg_us": sum(durs) / len(durs),
               "median_us": percentile(durs, 0.5), "p10_us": percentile(durs, 0.1),
               "p90_us": percentile(durs, 0.9), "min_us": min(durs), "max_us": max(durs),
               "companion_avg_us": side, "command": args.command}
    lines += ["", f"Timed steps only (the last {len(durs)} `{main}` launches, those of the K timed "
              "steps): avg {:.2f} us, median {:.2f}, p10 {:.2f}, p90 {:.2f}, min {:.2f}, max {:.2f}."
              .format(summary["avg_us"], summary["median_us"], summary["p10_us"], summary["p90_us"],
                      summary["min_us"], summary["max_us"])]
    if side:
        lines += ["", "Companion kernels per step (avg us): " +
                  ", ".join(f"{k} {v:.2f}" for k, v in side.items())]
    lines += ["", "Full kernel symbols:", ""] + [f"- `{o['kernel']}`" for o in out]
    with open(os.path.join(ROOT, "profiles", name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", name + ".json"), "w") as f:
        json.dump(summary, f, indent=1)
    print(os.path.join("profiles", name + ".md"), json.dumps(summary))


def summarize_timeline(args, w, variant):
    """Kernel timeline of the K timed steps of a `--only-run` trace: how much
    of the gather copies' time ran beside a GEMM launch, and the dispatches of
    the last two steps with their start and end times."""
    disp = _csv_rows(args.summarize_timeline, "kernel_trace.csv")
    disp = [r for r in disp if "rocclr" not in r["Kernel_Name"]]
    disp.sort(key=lambda r: int(r["Start_Timestamp"]))
    gathers = [i for i, r in enumerate(disp) if _short(r["Kernel_Name"]) == "gather_kernel"]
    disp = disp[:gathers[-3]]   # the 3 calibration copies run last
    main = next(k for k in MAIN_KERNELS if any(_short(r["Kernel_Name"]) == k for r in disp))
    gemm_idx = [i for i, r in enumerate(disp) if _short(r["Kernel_Name"]) == main]
    k_launches = args.steps * args.launches_per_step
    first = gemm_idx[-k_launches]
    # the timed steps start with the copy that feeds their first GEMM
    lo = max([i for i in range(first) if _short(disp[i]["Kernel_Name"]) == "gather_kernel"] or [first])
    window = disp[lo:]
    iv = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"])) for r in window]
    t0 = iv[0][0]
    gemm_iv = sorted((a, b) for a, b, k in iv if k == main)
    copy_iv = [(a, b) for a, b, k in iv if k == "gather_kernel"]

    def overlap(a, b):
        return sum(max(0, min(b, y) - max(a, x)) for x, y in gemm_iv)

    copy_ns = sum(b - a for a, b in copy_iv)
    copy_beside = sum(overlap(a, b) for a, b in copy_iv)
    wall_us = (max(b for _, b, _ in iv) - t0) / 1e3
    summary = {"workload": w.name, "variant": variant, "steps": args.steps, "step_us": wall_us / args.steps,
               "gemm_launches": len(gemm_iv), "copies": len(copy_iv),
               "copy_us_per_step": copy_ns / 1e3 / args.steps,
               "copy_us_beside_gemm_per_step": copy_beside / 1e3 / args.steps,
               "copy_frac_beside_gemm": copy_beside / copy_ns if copy_ns else 0.0,
               "gemm_us_per_step": sum(b - a for a, b in gemm_iv) / 1e3 / args.steps,
               "kernel_sha": kernel_source_sha(), "command": args.command}
    name = f"timeline_{w.name}_{variant}"
    lines = [f"# rocprofv3 kernel timeline: {w.name}, {variant} path", "", f"command: `{args.command}`", "",
             f"Over the {args.steps} timed steps: {summary['step_us']:.1f} us per step; gather copies "
             f"{summary['copy_us_per_step']:.1f} us per step, of which {summary['copy_us_beside_gemm_per_step']:.1f} us "
             f"({100 * summary['copy_frac_beside_gemm']:.0f}%) ran while a `{main}` launch was running; "
             f"GEMM launches {summary['gemm_us_per_step']:.1f} us per step (summed over launches, which may overlap).",
             "", "Dispatches of the last two steps (us from the first listed):", "",
             "| kernel | stream | start | end | duration |", "|---|---|---|---|---|"]
    per_step = max(1, len(window) // args.steps)
    for r in window[-2 * per_step:]:
        a, b = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        base = int(window[-2 * per_step]["Start_Timestamp"])
        lines.append(f"| {_short(r['Kernel_Name'])} | {r.get('Stream_Id', r.get('Queue_Id', ''))} | "
                     f"{(a - base) / 1e3:.1f} | {(b - base) / 1e3:.1f} | {(b - a) / 1e3:.1f} |")
    with open(os.path.join(ROOT, "profiles", name + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", name + ".json"), "w") as f:
        json.dump(summary, f, indent=1)
    print(os.path.join("profiles", name + ".md"), json.dumps(summary))


def summarize_traffic(args, w, variant):
    fetch_rows = _csv_rows(args.summarize_traffic[0], "counter_collection.csv")
    write_rows = _csv_rows(args.summarize_traffic[1], "counter_collection.csv")

    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            k = _short(r.get("Kernel_Name", ""))
            disp = r.get("Dispatch_Id")
            acc.setdefault(k, {}).setdefault(disp, 0.0)
            acc[k][disp] += float(r.get("Counter_Value", 0) or 0)
        out = {}
        for k, v in acc.items():
            ids = sorted(v, key=lambda x: int(x))
            if k == "gather_kernel":
                ids = ids[-3:]   # the 3 calibration copies run last
            out[k] = sum(v[i] for i in ids) / len(ids)   # KiB per dispatch
        return out

    fetch = per_kernel(fetch_rows, "FETCH_SIZE")
    write = per_kernel(write_rows, "WRITE_SIZE")
    copy_bytes = w.gather_bytes()
    # the gather copy reads and writes exactly m*k*elem bytes
    f_scale = copy_bytes / (fetch["gather_kernel"] * 1024.0)
    w_scale = copy_bytes / (write["gather_kernel"] * 1024.0)
    main = next(k for k in MAIN_KERNELS if k in fetch)
    fb = fetch[main] * 1024.0 * f_scale
    wb = write[main] * 1024.0 * w_scale
    extra = {}
    for key in ("splitk_reduce_kernel", "skinny_reduce_kernel"):
        if key in fetch:
            extra = {"reduce_kernel": key, "reduce_fetch_bytes": fetch[key] * 1024.0 * f_scale,
                     "reduce_write_bytes": write[key] * 1024.0 * w_scale}
    if "transpose16_kernel" in fetch:
        extra["transpose_fetch_bytes"] = fetch["transpose16_kernel"] * 1024.0 * f_scale
        extra["transpose_write_bytes"] = write["transpose16_kernel"] * 1024.0 * w_scale
    d = {"workload": w.name, "variant": variant, "kernel": main,
         "kernel_sha": kernel_source_sha(),
         "fetch_kib_raw": fetch[main], "write_kib_raw": write[main],
         "copy_fetch_kib_raw": fetch["gather_kernel"], "copy_write_kib_raw": write["gather_kernel"],
         "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
         "hbm_bytes_per_launch": fb + wb, "fetch_bytes_per_launch": fb,
         "write_bytes_per_launch": wb, "algorithmic_bytes": w.algorithmic_bytes(),
         "command": args.command, **extra}
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}_{variant}.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(path, json.dumps(d))


# ------------------------------------------------------------------ measuring
class Bench:
    """Inputs of one workload on the GPU plus the timing helpers."""

    def __init__(self, w, torch, agmm, I, np):
        self.w, self.torch, self.agmm, self.I, self.np = w, torch, agmm, I, np
        self.dev = torch.device("cuda:0")
        self.tdt = {0: torch.bfloat16, 1: torch.float16, 2: torch.float32}[w.dtype]
        itype = {0: np.int16, 1: np.int16, 2: np.int32}[w.dtype]
        t0 = time.time()
        self.shards_np, self.B_np = I.make_inputs(w)

        def up(bits):
            return torch.from_numpy(bits.view(itype)).view(self.tdt).to(self.dev)

        # Enough independent buffer sets that a step never finds its operands
        # in the 256 MB MALL from the previous step.
        self.nsets = max(1, min(32, math.ceil(2 * MALL_BYTES / w.algorithmic_bytes())))
        base_shards = [up(s) for s in self.shards_np]
        base_B = up(self.B_np)
        self.sets = []
        for i in range(self.nsets):
            sh = base_shards if i == 0 else [s.clone() for s in base_shards]
            Bt = base_B if i == 0 else base_B.clone()
            C = torch.empty((w.m, w.n_local), dtype=self.tdt, device=self.dev)
            self.sets.append((sh, Bt, C))
        self.gen_s = time.time() - t0
        self.stream = torch.cuda.current_stream()

    def settings(self, variant):
        w = self.w
        return {"pvalue": w.pvalue or 2, "nbuf": w.nbuf or 2} if variant == "staged" else {}

    def plan(self, variant, **extra):
        w = self.w
        st = {**self.settings(variant), **extra}
        return self.agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                              variant=variant, **st)

    def runner(self, plan):
        def run(i, s):
            sh, Bt, C = self.sets[i % self.nsets]
            plan.run(sh, Bt, C, stream=s)
        return run

    def warm(self, run, warmup, settle=True):
        torch = self.torch
        for i in range(warmup):
            run(i, self.stream)
        torch.cuda.synchronize()
        n, t0 = 0, time.time()
        while settle and time.time() - t0 < SETTLE_S:
            run(n, self.stream)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return n

    def eager_steps(self, run, steps):
        """K eager steps with an event before each and after the last: total
        ms per step (first to last event) and the per-step times."""
        torch = self.torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(self.stream)
        for i in range(steps):
            run(i, self.stream)
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return evs[0].elapsed_time(evs[-1]) / steps, per

    def graph_steps(self, run, steps, replays=10):
        """Capture `steps` calls into one HIP graph, replay it untimed until the
        clocks settle, then time `replays` replays one by one: ms per call of
        the first timed replay, and the per-call means of every replay."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    run(i, side)
        torch.cuda.synchronize()
        t0 = time.time()
        while time.time() - t0 < SETTLE_S / 2:   # untimed replays until the clocks have settled
            g.replay()
            torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
        evs[0].record(cur)
        for r in range(replays):
            g.replay()
            evs[r + 1].record(cur)
        torch.cuda.synchronize()
        per = [evs[r].elapsed_time(evs[r + 1]) / steps for r in range(replays)]
        del g
        return per[0], per

    def graph_replays(self, run, steps):
        """One call per HIP graph, one graph per buffer set (the library
        takes one staged call of a plan per graph); the graphs are replayed
        untimed until the clocks settle, then `steps` timed replays back to
        back, rotating over the buffer sets as the other timings do: (mean
        ms per call, per-replay ms), or None if the library refuses the
        capture."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        try:
            for i in range(min(self.nsets, steps)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.stream(side):
                    with torch.cuda.graph(g, stream=side):
                        run(i, side)
                graphs.append(g)
        except self.agmm.AgmmError:
            torch.cuda.synchronize()
            return None
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        while time.time() - t0 < SETTLE_S / 2:
            graphs[n % len(graphs)].replay()
            n += 1
            torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(cur)
        for r in range(steps):
            graphs[r % len(graphs)].replay()
            evs[r + 1].record(cur)
        torch.cuda.synchronize()
        per = [evs[r].elapsed_time(evs[r + 1]) for r in range(steps)]
        del graphs
        return evs[0].elapsed_time(evs[steps]) / steps, per

    def kernel_ms(self, plan, run, steps):
        """The dominant kernel per launch: K more steps with the library's
        events around each GEMM launch (on the stream it runs on)."""
        agmm, torch = self.agmm, self.torch
        agmm.agmm_plan_timing_begin(plan.handle)
        for i in range(steps):
            run(i, self.stream)
        torch.cuda.synchronize()
        k_ms, k_launches = agmm.agmm_plan_timing_read(plan.handle)
        agmm.agmm_plan_timing_end(plan.handle)
        return k_ms / max(k_launches, 1), max(1, k_launches // max(steps, 1))

    def measure(self, variant, steps, warmup, eager=False, with_kernel=True, staged_graphs=False, **extra):
        """One plan, warmed up and settled; returns a dict of its timings."""
        plan = self.plan(variant, **extra)
        try:
            used = self.agmm.VARIANT_NAMES[plan.get("variant_used")]
            run = self.runner(plan)
            settle = self.warm(run, warmup)
            ms, per = self.eager_steps(run, steps)
            res = {"variant": used, "eager_ms": ms, "settle_steps": settle, "timing": "eager calls",
                   "ms": ms, "per_step": per, "tile": plan.get("tile"), "splits": plan.get("splits")}
            if with_kernel:
                res["kernel_ms"], res["launches_per_step"] = self.kernel_ms(plan, run, steps)
            # a graph holds at most one staged call of a plan (the library refuses
            # more): short staged steps are timed as K replays of a one-call
            # graph (where the library accepts the capture: at most as many
            # chunks as ring slots), the others as K-call graphs
            if not eager and ms < GRAPH_MAX_STEP_MS and used == "staged":
                got = self.graph_replays(run, steps)
                if got is not None:
                    res["ms"], res["per_step"] = got
                    res["timing"] = "K replays of a one-call HIP graph"
            elif not eager and used == "staged" and staged_graphs and \
                    plan.get("num_chunks") <= plan.get("num_slots"):
                # longer staged steps keep eager timing; the one-call-graph
                # form (only for the forms the library captures: at most as
                # many chunks as ring slots) is reported beside it: a graph
                # replaces the cross-stream event hops between calls
                got = self.graph_replays(run, steps)
                if got is not None:
                    res["one_call_graphs_ms"] = got[0]
            elif not eager and ms < GRAPH_MAX_STEP_MS:
                res["ms"], res["per_step"] = self.graph_steps(run, steps)
                res["timing"] = "HIP-graph replay of the K steps"
                if with_kernel and used in ("fused", "skinny"):
                    # a graph-timed fused or skinny step holds nothing but the
                    # dominant kernel (and its split-K reduction): its replay
                    # time per step is that kernel's duration, free of the
                    # per-launch event overhead of the eager hooks
                    res["kernel_ms_events"] = res["kernel_ms"]
                    res["kernel_ms"] = res["ms"] / res["launches_per_step"]
        finally:
            plan.close()
        return res

    def roofline(self, kernel_ms, launches_per_step, variant):
        w = self.w
        flops_per_launch = w.flops() / launches_per_step
        achieved = flops_per_launch / (kernel_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        traffic = traffic_from_profiles(w.name, variant)   # HBM bytes per launch
        ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte where the two roofs meet
        prof = trace_from_profiles(w.name, variant)
        if w.dtype != 2 and w.flops() / w.algorithmic_bytes() < ridge:
            # below the ridge (the skinny workload): bound by HBM on B
            bytes_per_launch = w.algorithmic_bytes() / launches_per_step
            gbs = bytes_per_launch / (kernel_ms * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                 "kernel_ms": round(kernel_ms, 5), "launches_per_step": launches_per_step,
                 "tflops": round(achieved, 2)}
            per_unit = bytes_per_launch
            unit_peak = PEAK_HBM_GBS * 1e9
        else:
            r = {"bound": "mfma" if w.dtype != 2 else "alu", "achieved": round(achieved, 2),
                 "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                 "traffic": traffic, "kernel_ms": round(kernel_ms, 5),
                 "launches_per_step": launches_per_step}
            per_unit = flops_per_launch
            unit_peak = peak * 1e12
        if prof is not None:
            # the GEMM launch the library times includes its split-K reduction,
            # not the transposed copy of B that precedes it
            us = prof["avg_us"] + sum(v for k, v in prof.get("companion_avg_us", {}).items()
                                      if k != "transpose16_kernel")
            r["profile"] = {"file": f"profiles/kernel_trace_{w.name}_{variant}.json",
                            "kernel_us": round(us, 2), "median_us": round(prof["median_us"], 2),
                            "frac": round(per_unit / (us * 1e-6) / unit_peak, 4)}
        return r


def step_stats(per):
    return {"median": round(percentile(per, 0.5), 5), "p10": round(percentile(per, 0.1), 5),
            "p90": round(percentile(per, 0.9), 5)}


def other_workload(wid, args, torch, agmm, I, np):
    """The `workloads` entry of another configuration: its default path (and
    for the staged configuration the fused and unfused paths as well)."""
    w = I.WORKLOADS[wid]
    b = Bench(w, torch, agmm, I, np)
    variants = [resolve_variant(w, None)]
    if w.variant == "staged":
        variants = ["staged", "fused", "unfused"]
    elif wid == 2:   # the 4 x 512 x 4096 -> 1024 configuration: reported fused and staged
        variants = ["fused", "staged"]
    out = {"workload": w.name, "buffer_sets": b.nsets}
    for v in variants:
        log(f"{w.name}: {v}")
        res = b.measure(v, args.steps, args.warmup, staged_graphs=True)
        tfl = w.flops() / (res["ms"] * 1e-3) / 1e12
        gbs = w.algorithmic_bytes() / (res["ms"] * 1e-3) / 1e9
        entry = {"ms_per_step": round(res["ms"], 5), "step_ms": step_stats(res["per_step"]),
                 **({"one_call_graphs_ms_per_step": round(res["one_call_graphs_ms"], 5)}
                    if "one_call_graphs_ms" in res else {}),
                 "timing": res["timing"], "tflops": round(tfl, 2),
                 "frac_mfma": round(tfl / PEAK_TFLOPS[w.dtype], 4),
                 "alg_GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                 "tile": res["tile"], "splits": res["splits"],
                 "roofline": b.roofline(res["kernel_ms"], res["launches_per_step"], res["variant"])}
        out[res["variant"]] = entry
    if "staged" in out and "unfused" in out:
        g = measure_gather(b, args)
        out["gather_ms"] = g["ms"] if g else None
        if g:
            out["hidden_gather_frac"] = round(
                (out["unfused"]["ms_per_step"] - out["staged"]["ms_per_step"]) / g["ms"], 4)
    del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def measure_gather(b, args):
    w, torch, agmm = b.w, b.torch, b.agmm
    if (w.k * w.elem_bytes) % 16:
        return None
    G = torch.empty((w.m, w.k), dtype=b.tdt, device=b.dev)
    gplan = b.plan("auto")
    try:
        def grun(i, s):
            gplan.gather(b.sets[i % b.nsets][0], G, stream=s)
        b.warm(grun, 3)
        ms, per = b.eager_steps(grun, max(10, args.steps))
        if ms < GRAPH_MAX_STEP_MS and not args.eager:
            ms, per = b.graph_steps(grun, max(10, args.steps))
    finally:
        gplan.close()
    payload = w.gather_bytes()
    del G
    return {"ms": round(ms, 5), "payload_GB_s": round(payload / (ms * 1e-3) / 1e9, 1),
            "traffic_GB_s": round(2 * payload / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(2 * payload / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, w, shards_np, B_np, I, np):
    """The oracle as it stands: a bounded sample of the benchmarked workload
    on every allowed host thread, then the small workloads whole on one
    thread and on all of them."""
    import oracle
    threads = oracle.num_threads()
    # bounded sample: whole output rows (all n_local columns, full k), grown
    # until one run of the oracle over them takes about --cpu-seconds
    rows, nrows, t_cpu = [0], 1, 0.0
    while True:
        sel = [int(r) for r in np.linspace(0, w.m - 1, nrows)]
        t1 = time.perf_counter()
        oracle.agmm_f64(shards_np, B_np, w.dtype, w.rhs_transpose, rows=sel)
        t_cpu = time.perf_counter() - t1
        rows = sel
        if t_cpu >= 0.8 * args.cpu_seconds or nrows >= w.m:
            break
        nrows = min(w.m, max(nrows * 2, int(nrows * args.cpu_seconds / max(t_cpu, 1e-3))))
    cpu_flops = 2.0 * len(rows) * w.k * w.n_local
    out = {"value": round(cpu_flops / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"{len(rows)} of {w.m} output rows of {w.name} (all {w.n_local} columns, "
                     f"full k={w.k}), {t_cpu:.2f} s incl. decoding B"}
    small = {}
    for wid in (1, 2, 3):
        ws = I.WORKLOADS[wid]
        sh, Bs = I.make_inputs(ws)
        entry = {}
        for nthr in (1, threads):
            oracle.set_threads(nthr)
            t1 = time.perf_counter()
            oracle.agmm_f64(sh, Bs, ws.dtype, ws.rhs_transpose)
            dt = time.perf_counter() - t1
            entry[f"threads_{nthr}"] = {"s": round(dt, 4), "GFLOP_s": round(ws.flops() / dt / 1e9, 3)}
        small[ws.name] = entry
    oracle.set_threads(threads)
    out["whole_workloads"] = small
    return out


def main():
    faulthandler.enable()   # a native crash prints the Python stack
    args = parse()
    if args.summarize_trace or args.summarize_traffic or args.summarize_timeline:
        from all_gather_gemm_agmm_amd import inputs as I
        w = I.WORKLOADS[args.workload]
        variant = resolve_variant(w, args.variant)
        if args.summarize_trace:
            summarize_trace(args, w, variant)
        if args.summarize_timeline:
            summarize_timeline(args, w, variant)
        if args.summarize_traffic:
            summarize_traffic(args, w, variant)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X only: the all-gather matmul here runs each "
              "peer's shard as a local HBM buffer, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import all_gather_gemm_agmm_amd as agmm
    from all_gather_gemm_agmm_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    agmm.load_library()
    torch.cuda.set_device(0)

    w = I.WORKLOADS[args.workload]
    variant = resolve_variant(w, args.variant)
    b = Bench(w, torch, agmm, I, np)
    log(f"{w.name}: inputs resident ({b.nsets} buffer sets)")

    if args.only_run:
        plan = b.plan(variant)
        try:
            run = b.runner(plan)
            b.warm(run, args.warmup, settle=not args.no_settle)
            ms, _ = b.eager_steps(run, args.steps)
            used = agmm.VARIANT_NAMES[plan.get("variant_used")]
        finally:
            plan.close()
        if (w.k * w.elem_bytes) % 16 == 0:
            G = torch.empty((w.m, w.k), dtype=b.tdt, device=b.dev)
            gp = b.plan("auto")
            for i in range(3):
                gp.gather(b.sets[i % b.nsets][0], G, stream=b.stream)
            torch.cuda.synchronize()
            gp.close()
        print(json.dumps({"workload": w.name, "variant": used, "ms_per_step": ms,
                          "gather_bytes": w.gather_bytes()}), flush=True)
        return

    # the benchmarked path: warmup, settle, exactly K timed steps
    res = b.measure(variant, args.steps, args.warmup, eager=args.eager)
    used = res["variant"]
    log(f"{used}: {res['ms']:.4f} ms/step ({res['timing']}), kernel {res['kernel_ms']:.4f} ms")
    ms_per_step = res["ms"]
    value = w.flops() / (ms_per_step * 1e-3) / 1e12
    roofline = b.roofline(res["kernel_ms"], res["launches_per_step"], used)

    gather = None
    variants_ms = None
    if not args.no_compare:
        log("gather")
        gather = measure_gather(b, args)
        # C plus the gathered operand from one call (agmm_run_gather_out), the
        # side copy on the gather kernel or on the SDMA engines
        if gather:
            G = torch.empty((w.m, w.k), dtype=b.tdt, device=b.dev)
            for label, extra in (("side_kernel", {"gather_out": 1, "copy_engine": 0}),
                                 ("side_sdma", {"gather_out": 1, "copy_engine": 1}),
                                 ("sequential", {"gather_out": 2}), ("auto", {})):
                log(f"gather_out {label}")
                op = b.plan(variant, **extra)
                try:
                    def orun(i, s, op=op):
                        sh, Bt, C = b.sets[i % b.nsets]
                        op.run_gather_out(sh, Bt, C, G, stream=s)
                    b.warm(orun, 2)
                    ms, _ = b.eager_steps(orun, max(5, args.steps // 2))
                finally:
                    op.close()
                gather["gather_out_ms_" + label] = round(ms, 5)
            del G
        # the same problem through the other paths (overlap accounting)
        variants_ms = {}
        for v in ("fused", "staged", "staged_sdma", "unfused", "skinny"):
            if v == "skinny" and (w.dtype == 2 or w.m > 1024):
                continue
            if v in ("staged", "staged_sdma", "unfused") and (w.k * w.elem_bytes) % 16:
                continue
            log(f"variant {v}")
            extra = {"copy_engine": 1} if v == "staged_sdma" else {}
            r = b.measure(v.split("_")[0], max(5, args.steps // 2), 2, eager=args.eager,
                          with_kernel=False, **extra)
            variants_ms[v] = round(r["ms"], 5)
        if "unfused" in variants_ms and "staged" in variants_ms:
            variants_ms["unfused_over_staged"] = round(variants_ms["unfused"] / variants_ms["staged"], 4)
            if gather:
                variants_ms["hidden_gather_frac"] = round(
                    (variants_ms["unfused"] - variants_ms["staged"]) / gather["ms"], 4)

    shards_np, B_np, gen_s, nsets = b.shards_np, b.B_np, b.gen_s, b.nsets
    del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    workloads = []
    for wid in [int(x) for x in args.also.split(",") if x.strip()]:
        if wid == args.workload:
            continue
        workloads.append(other_workload(wid, args, torch, agmm, I, np))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cpu = cpu_baseline(args, w, shards_np, B_np, I, np)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "timing": res["timing"], "settle_steps": res["settle_steps"],
        "eager_ms_per_step": round(res["eager_ms"], 5), "step_ms": step_stats(res["per_step"]),
        "dtype": I.DTYPE_NAMES[w.dtype], "data": "synthetic (seeded, N(0,1/sqrt(k)) or U[-1,1])",
        "config": {**w.describe(), "variant": used, "tile": res["tile"], "splits": res["splits"],
                   "buffer_sets": nsets},
        "frac_of_peak": round(value / PEAK_TFLOPS[w.dtype], 4),
        "roofline": roofline, "gather": gather, "variants_ms": variants_ms,
        "workloads": workloads, "cpu_baseline": cpu, "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
