#!/usr/bin/env python3
"""Benchmark of the all-gather matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--variant auto]

One step = one agmm_run (the whole hot path: gather/slot sync/tile schedule/
MFMA GEMM/epilogue, as the chosen variant does them) over one batch of seeded
synthetic inputs already resident in HBM.  Prints ONE JSON line.

value      : 2*m*k*n_local / (wall time per step), TFLOP/s, timed with events
             around exactly K steps replayed from one HIP graph (--eager: K
             eager calls; the eager time is reported either way).  Before the
             timed region: W warmup steps, then untimed steps for SETTLE_S of
             wall time (the clocks' ramp; reported as settle_steps).
roofline   : the dominant kernel (the MFMA GEMM, with its split-K reduction
             when it has one) timed per launch with HIP events on the stream
             it is launched on, against the MI355X dense bf16/fp16 MFMA peak
             (2.5 PFLOP/s), or against HBM (8 TB/s, algorithmic bytes) for
             workloads below the ridge point (the skinny one).
gather     : the gather copy alone (agmm_gather) on the same shards, GB/s of
             payload (m*k*elem) and of HBM traffic (read + write).
variants_ms: the same problem through the fused, staged and unfused paths.
cpu_baseline: the CPU oracle on a bounded sample of output rows (rank 0).
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--variant", default=None, help="auto|fused|staged|unfused|skinny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as K eager calls instead of one replay of a HIP graph "
                         "holding them (the eager figure is always reported as eager_ms_per_step)")
    ap.add_argument("--only-run", action="store_true",
                    help="warmup + K steps of the main path, then 3 gather copies of the same "
                         "shards (the known-size copy that calibrates HBM counters); for profilers")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/ summary of a rocprofv3 --kernel-trace --stats CSV run")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ traffic summary from rocprofv3 --pmc FETCH_SIZE and "
                         "--pmc WRITE_SIZE CSV runs of --only-run")
    ap.add_argument("--command", default="", help="profiler command line, recorded in summaries")
    return ap.parse_args()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("gemm_mfma.hip", "skinny.hip", "gather_f32.hip", "agmm_kernels.h"):
        with open(os.path.join(ROOT, "all_gather_gemm_agmm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def _short(name: str) -> str:
    for key in ("gemm_m16_kernel", "gemm_mfma_kernel", "skinny_fullk_kernel", "splitk_reduce_kernel",
                "gather_kernel", "gemm_f32_kernel"):
        if key in name:
            return key
    return name[:48]


def summarize_trace(args, w, variant):
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
    lines += ["", "Full kernel symbols:", ""] + [f"- `{o['kernel']}`" for o in out]
    path = os.path.join(ROOT, "profiles", name + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


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
    main = next(k for k in ("gemm_m16_kernel", "gemm_mfma_kernel", "skinny_fullk_kernel", "gemm_f32_kernel")
                if k in fetch)
    fb = fetch[main] * 1024.0 * f_scale
    wb = write[main] * 1024.0 * w_scale
    extra = {}
    if "splitk_reduce_kernel" in fetch:
        extra = {"reduce_fetch_bytes": fetch["splitk_reduce_kernel"] * 1024.0 * f_scale,
                 "reduce_write_bytes": write["splitk_reduce_kernel"] * 1024.0 * w_scale}
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


GRAPH_MAX_STEP_MS = 0.25
# After the W warmup steps, untimed steps continue until this much wall time
# has passed: the GPU's clocks take more than ~10 ms of load to settle, and a
# short timed region would otherwise measure the ramp, not the kernels.
SETTLE_S = 0.2


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    faulthandler.enable()   # a native crash prints the Python stack
    args = parse()
    if args.summarize_trace or args.summarize_traffic:
        sys.path.insert(0, ROOT)
        from all_gather_gemm_agmm_amd import inputs as I
        w = I.WORKLOADS[args.workload]
        variant = args.variant or w.variant
        if variant == "auto":
            variant = "skinny" if (w.m <= 256 and w.dtype != 2) else "fused"
        if args.summarize_trace:
            summarize_trace(args, w, variant)
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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = I.WORKLOADS[args.workload]
    variant = args.variant or w.variant
    t0 = time.time()
    shards_np, B_np = I.make_inputs(w)
    tdt = {0: torch.bfloat16, 1: torch.float16, 2: torch.float32}[w.dtype]
    itype = {0: np.int16, 1: np.int16, 2: np.int32}[w.dtype]

    def up(bits):
        return torch.from_numpy(bits.view(itype)).view(tdt).to(dev)

    # Enough independent buffer sets that a step never finds its operands in
    # the 256 MB MALL from the previous step.
    ws_bytes = w.algorithmic_bytes()
    nsets = max(1, min(32, math.ceil(2 * MALL_BYTES / ws_bytes)))
    base_shards = [up(s) for s in shards_np]
    base_B = up(B_np)
    sets = []
    for i in range(nsets):
        sh = base_shards if i == 0 else [s.clone() for s in base_shards]
        Bt = base_B if i == 0 else base_B.clone()
        C = torch.empty((w.m, w.n_local), dtype=tdt, device=dev)
        sets.append((sh, Bt, C))
    gen_s = time.time() - t0
    log(f"{w.name}: inputs resident ({nsets} buffer sets)")

    settings = {}
    if variant == "staged":
        settings = {"pvalue": w.pvalue or 2, "nbuf": w.nbuf or 2}
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                     variant=variant, **settings)
    used = agmm.VARIANT_NAMES[plan.get("variant_used")]
    stream = torch.cuda.current_stream()

    def step(i, s=None):
        sh, Bt, C = sets[i % nsets]
        plan.run(sh, Bt, C, stream=s or stream)

    def graph_ms(run_one, count):
        """Capture `count` calls into one HIP graph, replay it once untimed,
        then time one replay between synchronisations: ms per call.  Every
        call's kernels are in the graph; only the host launch work is gone."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(count):
                    run_one(i, side)
        torch.cuda.synchronize()
        t_settle = time.time()
        while True:   # untimed replays until the clocks have settled
            g.replay()
            torch.cuda.synchronize()
            if time.time() - t_settle >= SETTLE_S / 2:
                break
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / count
        del g
        return ms

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    settle_steps = 0
    t_settle = time.time()
    while time.time() - t_settle < SETTLE_S:
        step(settle_steps)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warmup done ({used}; {settle_steps} settle steps)")

    # exactly K eager steps, nothing else recorded on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    eager_ms_per_step = ms_total / args.steps
    # the dominant kernel, per launch: another K steps with the library's
    # events around each GEMM launch (kept out of the timed steps above: on
    # the staged path they sit between the chunk launches of two streams)
    k_ms, k_launches = 0.0, 0
    if not args.only_run:
        agmm.agmm_plan_timing_begin(plan.handle)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        k_ms, k_launches = agmm.agmm_plan_timing_read(plan.handle)
        agmm.agmm_plan_timing_end(plan.handle)
    # Launch-bound steps (short ones, where eager calls measure the host's
    # call overhead) are timed as exactly K steps replayed from one HIP graph;
    # longer steps keep the eager timing, which those workloads have been
    # measured with (a graph-timed run of the largest workload crashed the
    # process and is not used until that crash is understood).
    use_graph = not args.eager and not args.only_run and eager_ms_per_step < GRAPH_MAX_STEP_MS
    log(f"eager {eager_ms_per_step:.4f} ms/step; timing {'graph' if use_graph else 'eager'}")
    ms_per_step = graph_ms(step, args.steps) if use_graph else eager_ms_per_step
    log("timed steps done")
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12

    if args.only_run:
        if (w.k * w.elem_bytes) % 16 == 0:
            G = torch.empty((w.m, w.k), dtype=tdt, device=dev)
            for i in range(3):
                plan.gather(sets[i % nsets][0], G, stream=stream)
            torch.cuda.synchronize()
        print(json.dumps({"workload": w.name, "variant": used, "ms_per_step": ms_per_step,
                          "gather_bytes": w.gather_bytes()}), flush=True)
        plan.close()
        return

    # dominant kernel: the GEMM launches (one per step, or one per chunk when staged)
    launches_per_step = max(1, k_launches // max(args.steps, 1))
    avg_launch_ms = k_ms / max(k_launches, 1)
    flops_per_launch = flops / launches_per_step
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = traffic_from_profiles(w.name, used)
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop per byte where the two roofs meet
    if w.dtype != 2 and w.flops() / w.algorithmic_bytes() < ridge:
        # below the ridge (the skinny workload): bound by HBM on B
        bytes_per_launch = w.algorithmic_bytes() / launches_per_step
        gbs = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel_ms": round(avg_launch_ms, 5), "launches_per_step": launches_per_step,
                    "tflops": round(achieved, 2)}
    else:
        roofline = {"bound": "mfma" if w.dtype != 2 else "alu", "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": traffic, "kernel_ms": round(avg_launch_ms, 5),
                    "launches_per_step": launches_per_step}

    # gather copy alone
    gather = None
    if (w.k * w.elem_bytes) % 16 == 0:
        G = torch.empty((w.m, w.k), dtype=tdt, device=dev)
        gplan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose)
        for i in range(3):
            gplan.gather(sets[i % nsets][0], G, stream=stream)
        torch.cuda.synchronize()

        def grun(i, s):
            gplan.gather(sets[i % nsets][0], G, stream=s)

        if use_graph:
            g_ms = graph_ms(grun, max(10, args.steps))
        else:
            gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gsteps = max(10, args.steps)
            gs.record(stream)
            for i in range(gsteps):
                grun(i, stream)
            ge.record(stream)
            torch.cuda.synchronize()
            g_ms = gs.elapsed_time(ge) / gsteps
        payload = w.gather_bytes()
        gather = {"ms": round(g_ms, 5), "payload_GB_s": round(payload / (g_ms * 1e-3) / 1e9, 1),
                  "traffic_GB_s": round(2 * payload / (g_ms * 1e-3) / 1e9, 1),
                  "frac_hbm": round(2 * payload / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        gplan.close()
        # C plus the gathered operand from one call (agmm_run_gather_out), the
        # side copy on the gather kernel or on the SDMA engines
        if not args.no_compare:
            for ce in (0, 1):
                log(f"gather_out copy_engine={ce}")
                op = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype,
                               w.rhs_transpose, variant=variant, copy_engine=ce, **settings)
                sh0, B0, C0 = sets[0]
                op.run_gather_out(sh0, B0, C0, G, stream=stream)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                nst = max(5, args.steps // 2)
                e0.record(stream)
                for i in range(nst):
                    sh, Bt, C = sets[i % nsets]
                    op.run_gather_out(sh, Bt, C, G, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                gather["gather_out_ms_" + ("sdma" if ce else "kernel")] = round(e0.elapsed_time(e1) / nst, 5)
                op.close()
        del G

    # the same problem through the other paths (overlap accounting)
    variants_ms = None
    if not args.no_compare:
        variants_ms = {}
        for v in ("fused", "staged", "staged_sdma", "unfused", "skinny"):
            if v == "skinny" and (w.dtype == 2 or w.m > 1024):
                continue
            if v in ("staged", "staged_sdma", "unfused") and (w.k * w.elem_bytes) % 16:
                continue
            st = {"pvalue": w.pvalue or 2, "nbuf": w.nbuf or 2} if v.startswith("staged") else {}
            if v == "staged_sdma":
                st["copy_engine"] = 1   # chunk copies after the first on the SDMA engines
            log(f"variant {v}")
            vp = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype,
                           w.rhs_transpose, variant=v.split("_")[0], **st)

            def vrun(i, s, vp=vp):
                sh, Bt, C = sets[i % nsets]
                vp.run(sh, Bt, C, stream=s)

            for i in range(2):
                vrun(i, stream)
            torch.cuda.synchronize()
            nst = max(5, args.steps // 2)
            if use_graph:
                variants_ms[v] = round(graph_ms(vrun, nst), 5)
            else:
                vs, ve = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                vs.record(stream)
                for i in range(nst):
                    vrun(i, stream)
                ve.record(stream)
                torch.cuda.synchronize()
                variants_ms[v] = round(vs.elapsed_time(ve) / nst, 5)
            vp.close()
        if "unfused" in variants_ms and "staged" in variants_ms:
            variants_ms["unfused_over_staged"] = round(variants_ms["unfused"] / variants_ms["staged"], 4)
        if gather and "unfused" in variants_ms and "staged" in variants_ms:
            variants_ms["hidden_gather_frac"] = round(
                (variants_ms["unfused"] - variants_ms["staged"]) / gather["ms"], 4)

    plan.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        import oracle
        # bounded sample: whole output rows (all n_local columns, full k),
        # grown until about --cpu-seconds of oracle work.
        rows = [0]
        t_cpu = 0.0
        nrows = 1
        while True:
            sel = [int(r) for r in np.linspace(0, w.m - 1, nrows)]
            t1 = time.time()
            oracle.agmm_f64(shards_np, B_np, w.dtype, w.rhs_transpose, rows=sel)
            t_cpu = time.time() - t1
            rows = sel
            if t_cpu > args.cpu_seconds / 4 or nrows >= w.m:
                break
            nrows = min(w.m, max(nrows * 2, int(nrows * (args.cpu_seconds / 4) / max(t_cpu, 1e-3))))
        cpu_flops = 2.0 * len(rows) * w.k * w.n_local
        cpu = {"value": round(cpu_flops / t_cpu / 1e12, 6), "unit": "TFLOP/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{len(rows)} of {w.m} output rows (all {w.n_local} columns, full k={w.k}), "
                         f"{t_cpu:.2f} s incl. decoding B"}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "timing": "one HIP-graph replay of the K steps" if use_graph else "eager calls",
        "settle_steps": settle_steps,
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "dtype": I.DTYPE_NAMES[w.dtype], "data": "synthetic (seeded, N(0,1/sqrt(k)) or U[-1,1])",
        "config": {**w.describe(), "variant": used, "buffer_sets": nsets},
        "frac_of_peak": round(value / PEAK_TFLOPS[w.dtype], 4),
        "roofline": roofline, "gather": gather, "variants_ms": variants_ms,
        "cpu_baseline": cpu, "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
