"""MatMulNBits benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--prefill-config 3]

A step is one pass of the whole hot path over one batch of synthetic input:
every linear of the workload (read activations, stream the packed int4
codes, scales and zero points, unpack, dequantize, contract, write outputs),
issued as one grouped launch. The headline workload is the Qwen3-0.6B-shaped
decode step (197 GEMVs: 28 layers x 7 projections + the LM head, M = 1,
block 32, fp16 activations). The same run also times the Qwen3-1.7B-shaped
prefill (196 GEMMs at M = 410) for the TFLOP/s half of the metric.

Inputs are resident in HBM before timing starts; the step rotates over
enough replicas of the weights to exceed the 256 MB last-level cache. Times
come from HIP events on the stream the kernels run on, over exactly K steps
bracketed by device synchronizations. Rank 0 prints one JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
LLC_BYTES = 256e6              # Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_COUNTERS_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")
# sources each measured kernel is built from (counter data is tied to them)
KERNEL_SOURCES = {
    "decode_grouped_kernel": ("mnb_gemv.hip", "mnb_decode.h", "mnb_device.h", "mnb_layout.h", "mnb_internal.h"),
    "gemm_grouped_kernel": ("mnb_gemm.hip", "mnb_device.h", "mnb_layout.h", "mnb_internal.h"),
    "decode_i8_grouped_kernel": ("mnb_int8.hip", "mnb_decode.h", "mnb_device.h", "mnb_layout.h",
                                 "mnb_internal.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "block_wise_int4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters for this kernel
    source, or None if absent or taken on a different source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(kernel_key.split(":")[0]):
        return None
    return rec.get("bytes_per_launch")


def stored_mfma_counters(kernel_key):
    """The matrix pipes' busy fraction and the clock measured with rocprofv3
    counters for this kernel source and workload, or None if absent or taken
    on a different source."""
    try:
        with open(MFMA_COUNTERS_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha(kernel_key.split(":")[0]):
        return None
    return rec


def record_traffic(fetch_csv, write_csv, probe_mib, workloads, command):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --copy-probe-mib) into HBM bytes per launch.

    Each counter is scaled by bytes / reading of the plain device copy of
    probe_mib MiB that the run made (the largest copy dispatch), so that the
    counters' units and what they count once are calibrated on the same box.
    Writes profiles/traffic.json and prints a markdown summary."""
    import csv

    probe = probe_mib << 20
    per = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch to calibrate {counter}")
        factors[counter] = probe / (max(copies) * 1024.0)
        for kernel in KERNEL_SOURCES:
            vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
            if vals:
                per.setdefault(kernel, {})[counter] = (sum(vals) / len(vals), len(vals))
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    lines = ["| kernel | workload | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | launches | "
             "HBM bytes/launch (calibrated) |", "|---|---|---:|---:|---:|---:|"]
    for kernel, vals in per.items():
        if "FETCH_SIZE" not in vals or "WRITE_SIZE" not in vals:
            continue
        fetch, n = vals["FETCH_SIZE"]
        write, _ = vals["WRITE_SIZE"]
        nbytes = int(round(fetch * 1024 * factors["FETCH_SIZE"] + write * 1024 * factors["WRITE_SIZE"]))
        key = f"{kernel}:{workloads[kernel]}"
        data[key] = {"bytes_per_launch": nbytes, "fetch_kib": round(fetch, 1), "write_kib": round(write, 1),
                     "fetch_factor": round(factors["FETCH_SIZE"], 5),
                     "write_factor": round(factors["WRITE_SIZE"], 5),
                     "source_sha": kernel_source_sha(kernel), "command": command}
        lines.append(f"| `{kernel}` | {workloads[kernel]} | {fetch:.1f} | {write:.1f} | {n} | {nbytes} |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"calibration ({probe_mib} MiB copy): FETCH_SIZE x {factors['FETCH_SIZE']:.5f}, "
          f"WRITE_SIZE x {factors['WRITE_SIZE']:.5f}")
    print("\n".join(lines))


def summarize_trace(trace_csv, bench_json, command, out_dir):
    """Kernel-trace summaries for profiles/: from a rocprofv3 --kernel-trace
    CSV of a bench.py run and that run's JSON line, one markdown file per
    timed workload (named kernel__workload), giving the trace's average
    duration over the timed launches beside bench.py's own HIP-event figure.

    A workload's grouped launches (first launch, warm-up, timed steps) run
    back to back, so they are the workload's run of consecutive dispatches
    of its kernel; runs of one kernel are matched to workloads in the order
    bench.py times them."""
    import csv

    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    runs = []  # (kernel name, [durations in us])
    for r in rows:
        name = r["Kernel_Name"]
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == name:
            runs[-1][1].append(d)
        else:
            runs.append((name, [d]))
    line = [ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    legs = [(res["config"]["workload"], res["roofline"], res["steps"], res["warmup"])]
    for key in ("prefill", "int8_mode"):
        if key in res:
            legs.append((res[key]["workload"], res[key]["roofline"], res[key]["steps"], res[key]["warmup"]))
    for name, leg in res.get("legs", {}).items():
        legs.append((name, leg["roofline"], leg["steps"], leg["warmup"]))
    totals = {}
    for name, durs in runs:
        t = totals.setdefault(name, [0, 0.0])
        t[0] += len(durs)
        t[1] += sum(durs)
    grand = sum(t[1] for t in totals.values())
    top = sorted(totals.items(), key=lambda kv: -kv[1][1])[:12]
    table = ["| kernel | calls | avg (us) | total (ms) | % GPU time |", "|---|---:|---:|---:|---:|"]
    for name, (n, tot) in top:
        table.append(f"| `{name}` | {n} | {tot / n:.2f} | {tot / 1e3:.1f} | {100 * tot / grand:.1f} |")
    used = set()
    written = []
    for workload, roof, steps, warmup in legs:
        kernel = roof["kernel"]
        # (template arguments name the tile variant in the trace; match on the kernel's base name)
        cand = [i for i, (n, d) in enumerate(runs) if i not in used and kernel in n and len(d) == warmup + steps]
        if not cand:
            log(f"[summarize] no run of {kernel} with {warmup + steps} launches for {workload}")
            continue
        i = cand[0]
        used.add(i)
        name, durs = runs[i]
        timed = durs[-steps:]
        avg = sum(timed) / len(timed)
        unit = roof["unit"]
        work = roof.get("algorithmic_flops_per_launch") if roof["bound"] == "mfma" else roof["algorithmic_bytes_per_launch"]
        rate = work / (avg * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
        text = [f"# {kernel} — {workload}", "",
                "Kernel trace on one MI355X, run from the repository root; the same run printed the bench JSON "
                "line whose figures are compared below.", "", "```", command, "```", "",
                f"Kernel `{name}`: {len(durs)} launches in this workload's run (first launch, {warmup - 1} more "
                f"warm-up, {steps} timed).", "",
                f"- trace, timed launches: average {avg:.2f} us (min {min(timed):.2f}, max {max(timed):.2f}); "
                f"first launch {durs[0]:.2f} us",
                f"- bench.py, same run (HIP events around the timed region / steps): {roof['launch_us']:.2f} us",
                f"- algorithmic {'FLOPs' if roof['bound'] == 'mfma' else 'bytes'} per launch: {work}",
                f"- at the trace average: {rate:.1f} {unit} = {100 * rate / roof['peak']:.1f}% of {roof['peak']} {unit}",
                "", "Top kernels of the whole run:", ""] + table
        fname = os.path.join(out_dir, f"{kernel}__{workload}.md")
        with open(fname, "w") as f:
            f.write("\n".join(text) + "\n")
        written.append(fname)
        print(f"{fname}: trace {avg:.2f} us, bench {roof['launch_us']:.2f} us")
    # the next-row lines of the headline workload: the fused LM-head argmax
    # (two kernels per call, alternating) and the embedding gather
    def last(name_part, n):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if name_part in r["Kernel_Name"]]
        return d[-n:] if len(d) >= n else None
    steps = res["steps"]
    head_name = res["config"]["workload"]
    if "lm_head_argmax" in res:
        la = res["lm_head_argmax"]
        fused, finish = last("decode_argmax_kernel", steps), last("argmax_finish_kernel", steps)
        if fused and finish:
            f_avg, g_avg = sum(fused) / steps, sum(finish) / steps
            text = [f"# decode_argmax_kernel — {head_name} LM head", "",
                    "Kernel trace on one MI355X, run from the repository root; the same run printed the bench "
                    "JSON line whose lm_head_argmax figures are compared below.", "", "```", command, "```", "",
                    f"LM head {la['shape'][0]} x {la['shape'][1]}, the last {steps} calls of each kernel:", "",
                    f"- `decode_argmax_kernel` (the product with per-workgroup argmax slots): {f_avg:.2f} us",
                    f"- `argmax_finish_kernel` (reduces the slots): {g_avg:.2f} us",
                    f"- bench.py, same run, time per fused call (both launches, back to back): "
                    f"{la['fused_argmax']['us_per_call']} us; the plain product that writes the logits: "
                    f"{la['plain_gemv']['us_per_call']} us",
                    f"- algorithmic bytes per fused call: {la['fused_argmax']['algorithmic_bytes']}"]
            fname = os.path.join(out_dir, f"decode_argmax_kernel__{head_name}-lm-head.md")
            with open(fname, "w") as f:
                f.write("\n".join(text) + "\n")
            written.append(fname)
            print(f"{fname}: {f_avg:.2f} + {g_avg:.2f} us")
    if "embedding_gather" in res:
        eg = res["embedding_gather"]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
             if "embed_gather_kernel" in r["Kernel_Name"]]
        keys = [k for k in eg if k.startswith("tokens_")]
        per = len(d) // max(len(keys), 1)
        if keys and per >= steps:
            text = [f"# embed_gather_kernel — {head_name} embedding rows", "",
                    "Kernel trace on one MI355X, run from the repository root; the same run printed the bench "
                    "JSON line whose embedding_gather figures are compared below.", "", "```", command, "```", "",
                    f"Table {eg['vocab']} x {eg['hidden']} int8, {eg['out']} out; the last {steps} calls of each "
                    "size:", "", "| rows | trace avg (us) | bench us per call | algorithmic bytes | GB/s (trace) |",
                    "|---:|---:|---:|---:|---:|"]
            for i, k in enumerate(keys):
                seg = d[i * per:(i + 1) * per][-steps:]
                avg = sum(seg) / len(seg)
                text.append(f"| {k.split('_')[1]} | {avg:.2f} | {eg[k]['us_per_call']} | {eg[k]['algorithmic_bytes']} "
                            f"| {eg[k]['algorithmic_bytes'] / (avg * 1e-6) / 1e9:.1f} |")
            fname = os.path.join(out_dir, f"embed_gather_kernel__{head_name}-embedding.md")
            with open(fname, "w") as f:
                f.write("\n".join(text) + "\n")
            written.append(fname)
            print(f"{fname}: written")
    return written


def summarize_counters(counter_csv, bench_json, timing_json, command, out_path):
    """MFMA counters of the prefill kernel for profiles/: from a rocprofv3
    --pmc run (SQ_INSTS_MFMA, SQ_INSTS_VALU_MFMA_MOPS_F16,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE, GRBM_COUNT) of
    a bench run and that run's JSON line, per MFMA workload: the MFMA flops
    the counters count against the algorithmic flops, and the matrix pipes'
    busy fraction while the GPU is active. The clock comes from the launch
    time of the same workload in `timing_json`, a bench run without counters
    (counter collection serializes launches and inflates their times)."""
    import csv

    disp = {}
    for r in csv.DictReader(open(counter_csv)):
        if "gemm_grouped_kernel" not in r["Kernel_Name"]:
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    runs = []
    for k in sorted(disp):
        if runs and runs[-1][0] == disp[k]["name"] and runs[-1][2] == k - 1:
            runs[-1][1].append(disp[k])
            runs[-1][2] = k
        else:
            runs.append([disp[k]["name"], [disp[k]], k])
    line = [ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    legs = [(res["config"]["workload"], res["roofline"], res["steps"], res["warmup"])]
    if "prefill" in res:
        legs.append((res["prefill"]["workload"], res["prefill"]["roofline"], res["prefill"]["steps"],
                     res["prefill"]["warmup"]))
    for name, leg in res.get("legs", {}).items():
        legs.append((name, leg["roofline"], leg["steps"], leg["warmup"]))
    cus, simds = 256, 4
    tline = [ln for ln in open(timing_json).read().splitlines() if ln.startswith("{")][-1]
    tres = json.loads(tline)
    launch_us = {tres["config"]["workload"]: tres["roofline"]["launch_us"]}
    if "prefill" in tres:
        launch_us[tres["prefill"]["workload"]] = tres["prefill"]["roofline"]["launch_us"]
    for name, leg in tres.get("legs", {}).items():
        launch_us[name] = leg["roofline"]["launch_us"]
    text = ["# gemm_grouped_kernel — MFMA counters", "",
            "rocprofv3 counters of the prefill (MFMA) kernel, one MI355X, run from the repository root. Each "
            "value is per launch (the same in every timed launch). The clock column is GRBM_GUI_ACTIVE per XCD "
            "over the launch time bench.py measured for the same workload in a run without counters (counter "
            "collection serializes launches and inflates their times); the TFLOP/s column is that run's.", "",
            "```", command, "```", "",
            "Derivations: one `v_mfma_f32_16x16x32_f16` is 16384 flops, so MFMA flops = SQ_INSTS_MFMA x 16384 "
            "(and SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 gives the same); the matrix pipes' busy fraction = "
            "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs), i.e. the share of "
            "the GPU-active cycles in which an MFMA occupies a SIMD's matrix pipe.", "",
            "| workload | kernel | SQ_INSTS_MFMA | MFMA flops / algorithmic | MFMA_MOPS_F16 x 512 / MFMA flops | "
            "SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | busy fraction | clock (GHz) | TFLOP/s |",
            "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    used = set()
    records = {}
    for workload, roof, steps, warmup in legs:
        if roof["bound"] != "mfma":
            continue
        cand = [i for i, (n, d, _) in enumerate(runs) if i not in used and len(d) == warmup + steps]
        if not cand:
            log(f"[summarize] no counter run with {warmup + steps} launches for {workload}")
            continue
        i = cand[0]
        used.add(i)
        name, ds, _ = runs[i]
        d = ds[-1]
        flops = d["SQ_INSTS_MFMA"] * 16384
        gui = d["GRBM_GUI_ACTIVE"] / 8
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * cus * simds)
        t_us = launch_us.get(workload)
        clock = gui / (t_us * 1e-6) / 1e9 if t_us else float("nan")
        tflops = roof["algorithmic_flops_per_launch"] / (t_us * 1e-6) / 1e12 if t_us else float("nan")
        short = name.split("(")[0].replace("void mnb::", "")
        records[f"gemm_grouped_kernel:{workload}"] = {
            "source_sha": kernel_source_sha("gemm_grouped_kernel"), "mfma_busy_fraction": round(busy, 4),
            "clock_ghz": round(clock, 3), "mfma_flops_per_launch": flops, "command": command}
        text.append(f"| {workload} | `{short}` | {d['SQ_INSTS_MFMA']:.0f} | "
                    f"{flops / roof['algorithmic_flops_per_launch']:.4f} | "
                    f"{d['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512 / flops:.4f} | {d['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | "
                    f"{d['GRBM_GUI_ACTIVE']:.0f} | {busy:.3f} | {clock:.2f} | {tflops:.1f} |")
    text += ["", "MFMA flops above the algorithmic ones are the M padding of the last row tile (for example "
             "416 / 410 rows). The busy fraction is the MFMA utilisation at the clock the GPU actually ran; "
             "against the 2.5 PFLOP/s peak, which assumes 2.4 GHz, the roofline fraction is lower by the clock "
             "ratio. Under the heaviest MFMA load the clock settles lowest."]
    with open(out_path, "w") as f:
        f.write("\n".join(text) + "\n")
    with open(MFMA_COUNTERS_FILE, "w") as f:
        json.dump(records, f, indent=1, sort_keys=True)
        f.write("\n")
    print("\n".join(text))


def time_steps(fn_list, steps, warmup, torch, per_launch=False):
    """Run fn_list[i % R]() for warmup + steps and time the last `steps` with
    HIP events on the current stream (the stream the kernels run on).
    Returns (ms per step, list of per-call ms or None). With per_launch, an
    event pair also brackets every timed call (a diagnostic: each pair adds
    several microseconds between the launches it separates)."""
    R = len(fn_list)
    for i in range(warmup):
        fn_list[i % R]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)] if per_launch else None
    start.record()
    for i in range(steps):
        if marks:
            marks[i][0].record()
        fn_list[(warmup + i) % R]()
        if marks:
            marks[i][1].record()
    end.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in marks] if marks else None
    return start.elapsed_time(end) / steps, per


def leg_floor(steps, warmup, est_ms):
    """Warm-up and timed launches for a leg that is not the headline: at
    least 20 warm-up launches, and at least 40 timed ones or 50 ms of timed
    work, whatever --steps says (a short timed region of a long kernel is
    dominated by the first launches' clock ramp)."""
    timed = max(steps, 40, math.ceil(50.0 / max(est_ms, 1e-3)))
    return timed, max(warmup, 20)


def run_workload(cfg, steps, warmup, per_linear, torch, dev, launch_events=False, floor=False):
    from block_wise_int4_amd import mnb, workload

    t0 = time.time()
    log(f"[bench] {cfg.name}: quantizing and packing {len(cfg.linears)} linears on the GPU")
    base = workload.build_config(cfg, dev).linears
    algo = workload.algorithmic_bytes(cfg)
    flops = workload.flops(cfg)
    weight_bytes = sum(ld.pw.packed.numel() for ld in base)
    io_bytes = sum(ld.x.numel() * ld.x.element_size() + ld.y.numel() * ld.y.element_size() for ld in base)
    replicas = max(1, math.ceil(1.1e9 / (weight_bytes + io_bytes)))
    sets = [base] + [workload.replicate(cfg, base) for _ in range(replicas - 1)]
    plans = [workload.make_plan(cfg, s) for s in sets]
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: ready in {time.time() - t0:.1f}s, {replicas} replicas "
        f"({replicas * (weight_bytes + io_bytes) / 1e9:.2f} GB resident)")

    launches = mnb.mnb_plan_launches(plans[0])
    fns = [lambda p=p: mnb.mnb_gemm_grouped(p) for p in plans]
    # the first launch of the workload on its own (cold: nothing warmed up);
    # it counts as the first warm-up step
    first_ms, _ = time_steps(fns[:1], 1, 0, torch)
    if floor:
        steps, warmup = leg_floor(steps, warmup, first_ms)
    ms, _ = time_steps(fns, steps, max(warmup - 1, 0), torch)
    out = {"ms": ms, "bytes": algo, "flops": flops, "replicas": replicas, "launches_per_step": launches,
           "first_launch_ms": first_ms, "steps": steps, "warmup": warmup}
    if launches == 1:
        # the step is one launch, back to back: the region's time per step is
        # the kernel's average duration (launch to launch)
        out["launch_ms"] = ms
    log(f"[bench] {cfg.name}: grouped {ms * 1e3:.1f} us/step over {steps} steps after {warmup} "
        f"({launches} launches per step; first launch {first_ms * 1e3:.1f} us)")
    if launch_events:
        _, per = time_steps(fns, steps, warmup, torch, per_launch=True)
        srt = sorted(per)
        out["launch_ms_events"] = sum(per) / len(per)
        log(f"[bench] {cfg.name}: with an event pair around each launch: avg {out['launch_ms_events'] * 1e3:.1f} us "
            f"(min {srt[0] * 1e3:.1f}, median {srt[len(srt) // 2] * 1e3:.1f}, max {srt[-1] * 1e3:.1f})")
    if per_linear:
        # prefill calls: mnb_gemm, and the split-K call (one workspace, shared
        # by every call of the pass: they run one after another on one stream)
        ws = None
        if cfg.m > 1:
            need = max(mnb.mnb_gemm_split_k_workspace_bytes(cfg.m, ld.pw, 0) for ld in base)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def one_pass(s, split=False):
            def f():
                for ld in s:
                    if cfg.m == 1:
                        mnb.mnb_gemv(ld.x.reshape(-1), ld.pw, ld.y.reshape(-1))
                    elif split:
                        mnb.mnb_gemm_split_k(ld.x, ld.pw, ws, ld.y)
                    else:
                        mnb.mnb_gemm(ld.x, ld.pw, ld.y)
            return f

        def graphs_of(passes):
            # the calls captured once per replica set into a HIP graph and
            # replayed: the device-side cost of one call per linear, without
            # the host's per-call overhead
            out_g = []
            side = torch.cuda.Stream(dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            for f in passes:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    f()
                out_g.append(g)
            torch.cuda.synchronize()
            return out_g

        passes = [one_pass(s) for s in sets]
        pl_steps = max(3, steps // 4)
        out["per_linear_ms"], _ = time_steps(passes, pl_steps, min(warmup, 3), torch)
        graphs = graphs_of(passes)
        out["per_linear_graph_ms"], _ = time_steps([g.replay for g in graphs], max(pl_steps, 10),
                                                   max(3, min(warmup, 10)), torch)
        del graphs
        log(f"[bench] {cfg.name}: per-linear {out['per_linear_ms'] * 1e3:.1f} us/step issued from the host, "
            f"{out['per_linear_graph_ms'] * 1e3:.1f} us/step replayed from a graph")
        if cfg.m > 1:
            split_passes = [one_pass(s, True) for s in sets]
            graphs = graphs_of(split_passes)
            out["per_linear_split_graph_ms"], _ = time_steps([g.replay for g in graphs], max(pl_steps, 10),
                                                             max(3, min(warmup, 10)), torch)
            del graphs
            log(f"[bench] {cfg.name}: per-linear split-K {out['per_linear_split_graph_ms'] * 1e3:.1f} us/step "
                f"replayed from a graph")
        del ws
    del plans, sets, base
    torch.cuda.empty_cache()
    return out


def leg_record(cfg, res, kernel):
    """JSON object for one timed workload: throughput, its roofline against
    the bound that applies, and the per-linear schedules."""
    mb = cfg.m > 1
    launch_ms = res.get("launch_ms", res["ms"])
    if mb:
        achieved = res["flops"] / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "algorithmic_flops_per_launch": res["flops"]}
    else:
        achieved = res["bytes"] / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": stored_traffic(f"{kernel}:{cfg.name}"), "kernel": kernel,
                 "launch_us": round(launch_ms * 1e3, 2),
                 "launch_timing": "timed region / steps (one launch per step, back to back)",
                 "algorithmic_bytes_per_launch": res["bytes"]})
    counters = stored_mfma_counters(f"{kernel}:{cfg.name}") if mb else None
    if counters:
        # the same rate against the dense fp16 peak at the clock the counters
        # measured (256 CUs x 4096 flop per clock), as context for the
        # 2.4 GHz spec peak that `frac` uses
        at_clock = 256 * 4096 * counters["clock_ghz"] / 1e3
        roof["counters"] = {"mfma_busy_fraction": counters["mfma_busy_fraction"],
                            "clock_ghz": counters["clock_ghz"], "peak_at_clock": round(at_clock, 1),
                            "frac_at_clock": round(achieved / at_clock, 4),
                            "source": os.path.relpath(MFMA_COUNTERS_FILE, ROOT)}
    rec = {"workload": cfg.name, "M": cfg.m, "linears": len(cfg.linears), "block_size": cfg.block_size,
           "steps": res["steps"], "warmup": res["warmup"], "ms_per_step": round(res["ms"], 5),
           "first_launch_us": round(res["first_launch_ms"] * 1e3, 2), "schedule": "grouped",
           "launches_per_step": res["launches_per_step"], "replicas": res["replicas"], "roofline": roof}
    if mb:
        rec.update({"value": round(res["flops"] / (res["ms"] * 1e-3) / 1e12, 2), "unit": "TFLOP/s"})
    else:
        rec.update({"value": round(res["bytes"] / (res["ms"] * 1e-3) / 1e9, 2), "unit": "GB/s"})
    if "per_linear_ms" in res:
        def rate(ms):
            return round((res["flops"] / (ms * 1e-3) / 1e12) if mb else (res["bytes"] / (ms * 1e-3) / 1e9), 2)
        rec["per_linear"] = {"unit": rec["unit"], "host_issued_ms_per_step": round(res["per_linear_ms"], 5),
                             "host_issued": rate(res["per_linear_ms"]),
                             "graph_ms_per_step": round(res["per_linear_graph_ms"], 5),
                             "graph": rate(res["per_linear_graph_ms"])}
        if "per_linear_split_graph_ms" in res:
            rec["per_linear"]["split_k_graph_ms_per_step"] = round(res["per_linear_split_graph_ms"], 5)
            rec["per_linear"]["split_k_graph"] = rate(res["per_linear_split_graph_ms"])
    return rec


def run_lm_head_argmax(cfg, steps, warmup, torch, dev):
    """The workload's LM head alone: the fused greedy argmax (no logits
    written) against the plain decode product (logits written), one launch
    per step each, rotating over replicas past the last-level cache."""
    from block_wise_int4_amd import mnb, workload

    lin = [l for l in cfg.linears if l.proj == "lm_head"][0]
    ld = workload.build_linear(cfg, lin, dev)
    a = 2 if cfg.dtype == "f16" else 4
    nb = lin.k // cfg.block_size
    wbytes = lin.n * lin.k // 2 + lin.n * nb * a + (0 if cfg.symmetric else lin.n * ((nb + 1) // 2))
    reps = max(1, math.ceil(1.1e9 / ld.pw.packed.numel()))
    pws = [ld.pw] + [mnb.PackedWeight(ld.pw.packed.clone(), ld.pw.N, ld.pw.K, ld.pw.block_size, ld.pw.dtype,
                                      ld.pw.bits) for _ in range(reps - 1)]
    x = ld.x.reshape(-1)
    ws = mnb.argmax_workspace(dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    y = torch.empty(lin.n, dtype=ld.y.dtype, device=dev)
    # the greedy step's hand-over to the next input embedding: argmax, then
    # the gather of that token's row (three launches), against the product's
    # partial results reduced by the gather itself (two launches)
    from workloads import synth
    table, scales, _ = synth.embedding_inputs(2, lin.n, lin.k, 1)
    td, sd = torch.from_numpy(table).to(dev), torch.from_numpy(scales).to(dev)
    row = torch.empty((1, lin.k), dtype=ld.y.dtype, device=dev)
    def two_step(p):
        mnb.mnb_gemv_argmax(x, p, ws, index=idx)
        mnb.mnb_embed_gather(td, sd, idx, dtype=row.dtype, out=row)
    def handed_over(p):
        mnb.mnb_gemv_argmax(x, p, ws, partial=True)
        mnb.mnb_embed_gather_argmax(td, sd, ws, dtype=row.dtype, out=row, index=idx)
    kt, _ = time_steps([lambda p=p: two_step(p) for p in pws], steps, warmup, torch)
    kh, _ = time_steps([lambda p=p: handed_over(p) for p in pws], steps, warmup, torch)
    del td, sd
    kf, _ = time_steps([lambda p=p: mnb.mnb_gemv_argmax(x, p, ws, index=idx) for p in pws], steps, warmup, torch)
    kg, _ = time_steps([lambda p=p: mnb.mnb_gemv(x, p, y) for p in pws], steps, warmup, torch)
    bf = wbytes + lin.k * a + 8
    bg = wbytes + lin.k * a + lin.n * a
    log(f"[bench] {cfg.name} LM head {lin.n}x{lin.k}: fused argmax {kf * 1e3:.1f} us, plain {kg * 1e3:.1f} us; "
        f"argmax then embedding row {kt * 1e3:.1f} us, handed over {kh * 1e3:.1f} us")
    del pws
    torch.cuda.empty_cache()
    return {"shape": [lin.n, lin.k], "replicas": reps,
            "fused_argmax": {"us_per_call": round(kf * 1e3, 2), "launches_per_call": 2,
                             "algorithmic_bytes": bf, "GBps": round(bf / (kf * 1e-3) / 1e9, 1),
                             "frac_hbm": round(bf / (kf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "plain_gemv": {"us_per_call": round(kg * 1e3, 2), "launches_per_call": 1,
                           "algorithmic_bytes": bg, "GBps": round(bg / (kg * 1e-3) / 1e9, 1)},
            "argmax_to_embedding": {"two_step_us_per_call": round(kt * 1e3, 2), "two_step_launches": 3,
                                    "handed_over_us_per_call": round(kh * 1e3, 2), "handed_over_launches": 2,
                                    "embedding": [lin.n, lin.k], "note": "mnb_gemv_argmax + mnb_embed_gather "
                                    "against mnb_gemv_argmax (partial) + mnb_embed_gather_argmax"}}


def run_embed_gather(cfg, steps, warmup, torch, dev, token_counts=(410, 65536)):
    """Int8 embedding-row gather for the workload's vocabulary and width,
    float16 out: a prompt-sized call (410 rows) and a bandwidth-sized one,
    each rotating over two table copies and eight id sets so that rows come
    from HBM."""
    import numpy as np

    from block_wise_int4_amd import mnb
    from workloads import synth

    lin = [l for l in cfg.linears if l.proj == "lm_head"][0]
    vocab, hidden = lin.n, lin.k
    table, scales, _ = synth.embedding_inputs(1, vocab, hidden, 1)
    tables = [torch.from_numpy(table).to(dev) for _ in range(2)]
    sc = torch.from_numpy(scales).to(dev)
    rng = np.random.default_rng(5)
    res = {"vocab": vocab, "hidden": hidden, "out": "f16"}
    for tokens in token_counts:
        id_sets = [torch.from_numpy(rng.integers(0, vocab, size=tokens, dtype=np.int64)).to(dev) for _ in range(8)]
        out = torch.empty((tokens, hidden), dtype=torch.float16, device=dev)
        fns = [lambda t=t, i=i: mnb.mnb_embed_gather(t, sc, i, torch.float16, out=out)
               for i in id_sets for t in tables]
        k, _ = time_steps(fns, steps, warmup, torch)
        nbytes = tokens * hidden + tokens * 4 + tokens * 8 + tokens * hidden * 2
        log(f"[bench] embedding gather {tokens} x {hidden} of {vocab}: {k * 1e3:.1f} us")
        res[f"tokens_{tokens}"] = {"us_per_call": round(k * 1e3, 2), "algorithmic_bytes": nbytes,
                                   "GBps": round(nbytes / (k * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(nbytes / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del id_sets, out
    del tables
    torch.cuda.empty_cache()
    return res


def run_int8_mode(cfg, steps, warmup, torch, dev):
    """The decode workload in the int8 compute mode (activations quantized
    per block to int8 inside the kernel, integer dot products): the whole
    step as one grouped launch (mnb_plan_grouped_i8), rotating over replicas
    past the last-level cache; and, for context, one mnb_gemm_i8 call per
    linear replayed from a HIP graph. Bytes: the step's algorithmic bytes
    (codes, scales, zero points, activations and outputs)."""
    from block_wise_int4_amd import mnb, workload

    base = workload.build_config(cfg, dev).linears
    algo = workload.algorithmic_bytes(cfg)
    weight_bytes = sum(ld.pw.packed.numel() for ld in base)
    replicas = max(1, math.ceil(1.1e9 / weight_bytes))
    sets = [base] + [workload.replicate(cfg, base) for _ in range(replicas - 1)]
    dt = torch.float16 if cfg.dtype == "f16" else torch.float32
    plans = [mnb.mnb_plan_grouped([(ld.x.reshape(-1), ld.pw, ld.y) for ld in s], cfg.block_size, dt, int8=True)
             for s in sets]
    launches = mnb.mnb_plan_launches(plans[0])
    fns = [lambda p=p: mnb.mnb_gemm_grouped(p) for p in plans]
    first_ms, _ = time_steps(fns[:1], 1, 0, torch)
    ms, _ = time_steps(fns, steps, max(warmup - 1, 0), torch)
    gbs = algo / (ms * 1e-3) / 1e9
    log(f"[bench] {cfg.name} int8 compute mode: grouped {ms * 1e3:.1f} us/step ({gbs:.0f} GB/s, "
        f"{launches} launch per step)")

    def one_pass(s):
        def f():
            for ld in s:
                mnb.mnb_gemm_i8(ld.x.reshape(cfg.m, -1), ld.pw, None, ld.y.reshape(cfg.m, -1))
        return f
    passes = [one_pass(s) for s in sets]
    for f in passes:
        f()
    torch.cuda.synchronize()
    graphs = []
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    for f in passes:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    pl_ms, _ = time_steps([g.replay for g in graphs], max(10, steps // 4), max(3, min(warmup, 10)), torch)
    log(f"[bench] {cfg.name} int8 compute mode: per-linear {pl_ms * 1e3:.1f} us/step from a graph")
    del graphs, plans, sets, base
    torch.cuda.empty_cache()
    roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(f"decode_i8_grouped_kernel:{cfg.name}"), "kernel": "decode_i8_grouped_kernel",
            "launch_us": round(ms * 1e3, 2), "algorithmic_bytes_per_launch": algo}
    if launches == 1:
        roof["launch_timing"] = "timed region / steps (one launch per step, back to back)"
    return {"workload": cfg.name, "mode": "int8 activations (per-block symmetric, quantized in LDS), "
                                          "integer dot products",
            "schedule": "grouped", "launches_per_step": launches, "replicas": replicas, "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(ms, 5), "first_launch_us": round(first_ms * 1e3, 2),
            "value": round(gbs, 2), "unit": "GB/s", "roofline": roof,
            "per_linear": {"unit": "GB/s", "graph_ms_per_step": round(pl_ms, 5),
                           "graph": round(algo / (pl_ms * 1e-3) / 1e9, 2)}}


def run_int8_prefill(cfg, steps, warmup, torch, dev):
    """A prefill workload in the int8 compute mode: one mnb_gemm_i8 call per
    linear (the activation quantizer, then the int8 matrix-core product),
    issued back to back with one shared workspace. Rate: algorithmic
    operations (2 M N K) per second."""
    from block_wise_int4_amd import mnb, workload

    base = workload.build_config(cfg, dev).linears
    flops = workload.flops(cfg)
    need = max(mnb.mnb_gemm_i8_workspace_bytes(cfg.m, ld.pw.K, ld.pw.block_size) for ld in base)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def one_pass():
        for ld in base:
            mnb.mnb_gemm_i8(ld.x, ld.pw, ws, ld.y)
    first_ms, _ = time_steps([one_pass], 1, 0, torch)
    n = max(5, min(steps, int(200.0 / max(first_ms, 1e-3))))
    ms, _ = time_steps([one_pass], n, 2, torch)
    tops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {cfg.name} int8 compute mode: per-linear {ms * 1e3:.1f} us/step ({tops:.1f} TOP/s)")
    del base, ws
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "schedule": "per-linear mnb_gemm_i8 (quantize + int8 matrix-core product)",
            "launches_per_step": 2 * len(cfg.linears), "steps": n, "ms_per_step": round(ms, 5),
            "value": round(tops, 2), "unit": "TOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": 5000.0, "unit": "TOP/s",
                         "frac": round(tops / 5000.0, 4), "note": "int8 dense MFMA peak"}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, budget_s, runs=3):
    """The oracle (NumPy float64 dequantize + matmul) on the host cores, on a
    bounded prefix of the workload's linears: the prefix the first pass
    finishes within budget_s / runs, then the same prefix again, `runs`
    passes in all. Quantization is not timed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workloads import synth

    dt = np.float16 if cfg.dtype == "f16" else np.float32
    done_bytes, done_flops, first, used, sample = 0, 0, 0.0, [], []
    for lin in cfg.linears:
        if first >= budget_s / runs:
            break
        w, x = synth.linear_inputs(cfg, lin)
        n_rows = lin.n
        if lin.proj == "lm_head":
            n_rows = min(lin.n, 16384)   # a slice of the vocabulary keeps the sample bounded
            w = w[:n_rows]
        quantize = oracle.rtn_quantize_symmetric if cfg.symmetric else oracle.rtn_quantize
        q, s, zp = quantize(w, cfg.block_size, dt)
        t = time.perf_counter()
        oracle.matmul_nbits(x, q, zp, s, cfg.block_size)
        first += time.perf_counter() - t
        sample.append((x, q, zp, s))
        nb = lin.k // cfg.block_size
        a = 2 if cfg.dtype == "f16" else 4
        zp_bytes = 0 if cfg.symmetric else n_rows * ((nb + 1) // 2)
        done_bytes += n_rows * lin.k // 2 + n_rows * nb * a + zp_bytes + cfg.m * (lin.k + n_rows) * a
        done_flops += 2 * cfg.m * n_rows * lin.k
        used.append(f"{lin.proj}{'' if lin.layer < 0 else lin.layer}" + ("" if n_rows == lin.n else f"[:{n_rows}]"))
    times = [first]
    for _ in range(runs - 1):
        t = time.perf_counter()
        for x, q, zp, s in sample:
            oracle.matmul_nbits(x, q, zp, s, cfg.block_size)
        times.append(time.perf_counter() - t)
    times.sort()
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"median_s": times[len(times) // 2], "min_s": times[0], "bytes": done_bytes, "flops": done_flops,
            "cores": len(os.sched_getaffinity(0)), "blas_threads": blas, "cpu_model": cpu_model(), "runs": runs,
            "sample": f"{len(used)} of {len(cfg.linears)} linears in order ({used[0]}..{used[-1]}), "
                      f"{done_bytes / 1e6:.1f} MB algorithmic, {done_flops / 1e9:.1f} GFLOP; {runs} passes"}


def cpu_record(cb, mb):
    """cpu_baseline JSON object: throughput of the median pass (and of the
    fastest), in the workload's unit."""
    if mb:
        val = lambda t: round(cb["flops"] / t / 1e12, 5)  # noqa: E731
        unit = "TFLOP/s"
    else:
        val = lambda t: round(cb["bytes"] / t / 1e9, 4)  # noqa: E731
        unit = "GB/s"
    return {"value": val(cb["median_s"]), "unit": unit, "cores": cb["cores"], "kind": "oracle",
            "sample": cb["sample"], "best": val(cb["min_s"]), "median_s": round(cb["median_s"], 3),
            "min_s": round(cb["min_s"], 3), "blas_threads": cb["blas_threads"], "cpu_model": cb["cpu_model"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=1, help="headline workload (index into workloads.configs)")
    ap.add_argument("--prefill-config", type=int, default=3, help="prefill workload timed alongside; -1 = none")
    ap.add_argument("--extra-configs", default="2,4,5",
                    help="further workloads timed as legs of the line (comma-separated indices; '' = none)")
    ap.add_argument("--no-per-linear", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the LM-head argmax and embedding-gather lines")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8 compute-mode line")
    ap.add_argument("--launch-events", action="store_true",
                    help="also time each launch between its own event pair (diagnostic; logged, not reported)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work per workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size (counter calibration runs)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store HBM bytes per launch from two counter runs (no GPU needed)")
    ap.add_argument("--traffic-command", default="", help="the profiled command, stored with --record-traffic")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("COUNTER_CSV", "BENCH_JSON", "TIMING_JSON"),
                    help="write the MFMA counter summary for profiles/ from a --pmc run of bench (no GPU needed)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"),
                    help="write profiles/ summaries from a kernel trace of a bench run (no GPU needed)")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.traffic_command,
                           os.path.join(ROOT, "profiles", "gemm_grouped_kernel__mfma-counters.md"))
        return

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.traffic_command, os.path.join(ROOT, "profiles"))
        return

    from workloads import configs
    extra = [int(c) for c in args.extra_configs.split(",") if c.strip()]

    if args.record_traffic:
        wl = {"decode_grouped_kernel": configs.CONFIGS[args.config].name,
              "gemm_grouped_kernel": configs.CONFIGS[args.prefill_config].name,
              "decode_i8_grouped_kernel": configs.CONFIGS[args.config].name}
        record_traffic(*args.record_traffic, args.copy_probe_mib or 512, wl, args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_wise_int4_amd import mnb

    if not os.path.exists(mnb.LIB_PATH):
        from block_wise_int4_amd import build as _b
        _b.build()
    mnb.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {n} bytes read, {n} bytes written")
        ms_copy, _ = time_steps([lambda: b.copy_(a)], 10, 2, torch)
        copy_gbs = 2 * n / (ms_copy * 1e-3) / 1e9
        log(f"[bench] device copy of {args.copy_probe_mib} MiB: {ms_copy * 1e3:.1f} us = {copy_gbs:.0f} GB/s read+write")
        del a, b

    def kernel_of(c):
        return "decode_grouped_kernel" if c.m == 1 else "gemm_grouped_kernel"

    # headline: exactly --steps timed steps after --warmup
    cfg = configs.CONFIGS[args.config]
    dec = run_workload(cfg, args.steps, args.warmup, not args.no_per_linear, torch, dev, args.launch_events)
    head = leg_record(cfg, dec, kernel_of(cfg))
    gbs = dec["bytes"] / (dec["ms"] * 1e-3) / 1e9

    result = {
        "metric": "int4 MatMulNBits decode GB/s (M=1) & prefill TFLOP/s, % of MI355X roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,0.02) weights RTN-quantized on the GPU, N(0,1) activations)",
        "config": {
            "workload": cfg.name, "M": cfg.m, "linears": len(cfg.linears), "block_size": cfg.block_size,
            "symmetric": cfg.symmetric,
            "activations": cfg.dtype, "accumulate": "f32", "schedule": "grouped",
            "launches_per_step": dec["launches_per_step"], "replicas": dec["replicas"],
            "algorithmic_bytes_per_step": dec["bytes"],
            "first_launch_us": head["first_launch_us"],
        },
        "roofline": head["roofline"],
    }
    if "per_linear" in head:
        result["config"]["per_linear"] = head["per_linear"]

    if any(l.proj == "lm_head" for l in cfg.linears) and not args.no_next:
        result["lm_head_argmax"] = run_lm_head_argmax(cfg, args.steps, args.warmup, torch, dev)
        result["embedding_gather"] = run_embed_gather(cfg, args.steps, args.warmup, torch, dev)

    if not args.no_int8 and cfg.m == 1:
        result["int8_mode"] = run_int8_mode(cfg, args.steps, args.warmup, torch, dev)

    if args.prefill_config >= 0:
        pcfg = configs.CONFIGS[args.prefill_config]
        pre = run_workload(pcfg, args.steps, args.warmup, not args.no_per_linear, torch, dev, args.launch_events,
                           floor=True)
        result["prefill"] = leg_record(pcfg, pre, kernel_of(pcfg))
        if not args.no_int8 and pcfg.dtype == "f16":
            result["prefill"]["int8_mode"] = run_int8_prefill(pcfg, args.steps, args.warmup, torch, dev)

    legs = {}
    for ci in extra:
        ecfg = configs.CONFIGS[ci]
        res = run_workload(ecfg, args.steps, args.warmup, not args.no_per_linear, torch, dev, args.launch_events,
                           floor=True)
        legs[ecfg.name] = leg_record(ecfg, res, kernel_of(ecfg))
    if legs:
        result["legs"] = legs

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {cfg.name} (budget {args.cpu_budget:.0f}s)")
        result["cpu_baseline"] = cpu_record(cpu_baseline(cfg, args.cpu_budget), cfg.m > 1)
        if args.prefill_config >= 0:
            pcfg = configs.CONFIGS[args.prefill_config]
            log(f"[bench] cpu baseline: oracle on {pcfg.name}")
            result["prefill"]["cpu_baseline"] = cpu_record(cpu_baseline(pcfg, args.cpu_budget), True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
