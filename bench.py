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
# sources each measured kernel is built from (counter data is tied to them)
KERNEL_SOURCES = {
    "decode_grouped_kernel": ("mnb_gemv.hip", "mnb_device.h", "mnb_layout.h", "mnb_internal.h"),
    "gemm_grouped_kernel": ("mnb_gemm.hip", "mnb_device.h", "mnb_layout.h", "mnb_internal.h"),
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


def run_workload(cfg, steps, warmup, per_linear, torch, dev, launch_events=False):
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
    ms, _ = time_steps(fns, steps, warmup, torch)
    out = {"ms": ms, "bytes": algo, "flops": flops, "replicas": replicas, "launches_per_step": launches}
    if launches == 1:
        # the step is one launch, back to back: the region's time per step is
        # the kernel's average duration (launch to launch)
        out["launch_ms"] = ms
    log(f"[bench] {cfg.name}: grouped {ms * 1e3:.1f} us/step ({launches} launches per step)")
    if launch_events:
        _, per = time_steps(fns, steps, warmup, torch, per_launch=True)
        srt = sorted(per)
        out["launch_ms_events"] = sum(per) / len(per)
        log(f"[bench] {cfg.name}: with an event pair around each launch: avg {out['launch_ms_events'] * 1e3:.1f} us "
            f"(min {srt[0] * 1e3:.1f}, median {srt[len(srt) // 2] * 1e3:.1f}, max {srt[-1] * 1e3:.1f})")
    if per_linear:
        def one_pass(s):
            def f():
                for ld in s:
                    if cfg.m == 1:
                        mnb.mnb_gemv(ld.x.reshape(-1), ld.pw, ld.y.reshape(-1))
                    else:
                        mnb.mnb_gemm(ld.x, ld.pw, ld.y)
            return f
        pl_steps = max(3, steps // 4)
        out["per_linear_ms"], _ = time_steps([one_pass(s) for s in sets], pl_steps, min(warmup, 3), torch)
        log(f"[bench] {cfg.name}: per-linear {out['per_linear_ms'] * 1e3:.1f} us/step")
    del plans, sets, base
    torch.cuda.empty_cache()
    return out


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
    kf, _ = time_steps([lambda p=p: mnb.mnb_gemv_argmax(x, p, ws, index=idx) for p in pws], steps, warmup, torch)
    kg, _ = time_steps([lambda p=p: mnb.mnb_gemv(x, p, y) for p in pws], steps, warmup, torch)
    bf = wbytes + lin.k * a + 8
    bg = wbytes + lin.k * a + lin.n * a
    log(f"[bench] {cfg.name} LM head {lin.n}x{lin.k}: fused argmax {kf * 1e3:.1f} us, plain {kg * 1e3:.1f} us")
    del pws
    torch.cuda.empty_cache()
    return {"shape": [lin.n, lin.k], "replicas": reps,
            "fused_argmax": {"us_per_call": round(kf * 1e3, 2), "launches_per_call": 2,
                             "algorithmic_bytes": bf, "GBps": round(bf / (kf * 1e-3) / 1e9, 1),
                             "frac_hbm": round(bf / (kf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "plain_gemv": {"us_per_call": round(kg * 1e3, 2), "launches_per_call": 1,
                           "algorithmic_bytes": bg, "GBps": round(bg / (kg * 1e-3) / 1e9, 1)}}


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


def cpu_baseline(cfg, budget_s):
    """The oracle (NumPy float64 dequantize + matmul) on the host cores, on a
    bounded prefix of the workload's linears. Quantization is not timed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from workloads import synth

    dt = np.float16 if cfg.dtype == "f16" else np.float32
    done_bytes, done_flops, elapsed, used = 0, 0, 0.0, []
    for lin in cfg.linears:
        if elapsed >= budget_s:
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
        elapsed += time.perf_counter() - t
        nb = lin.k // cfg.block_size
        a = 2 if cfg.dtype == "f16" else 4
        zp_bytes = 0 if cfg.symmetric else n_rows * ((nb + 1) // 2)
        done_bytes += n_rows * lin.k // 2 + n_rows * nb * a + zp_bytes + cfg.m * (lin.k + n_rows) * a
        done_flops += 2 * cfg.m * n_rows * lin.k
        used.append(f"{lin.proj}{'' if lin.layer < 0 else lin.layer}" + ("" if n_rows == lin.n else f"[:{n_rows}]"))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"seconds": elapsed, "bytes": done_bytes, "flops": done_flops, "threads": threads,
            "sample": f"{len(used)} of {len(cfg.linears)} linears in order ({used[0]}..{used[-1]}), "
                      f"{done_bytes / 1e6:.1f} MB algorithmic"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=1, help="headline workload (index into workloads.configs)")
    ap.add_argument("--prefill-config", type=int, default=3, help="prefill workload timed alongside; -1 = none")
    ap.add_argument("--no-per-linear", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the LM-head argmax and embedding-gather lines")
    ap.add_argument("--launch-events", action="store_true",
                    help="also time each launch between its own event pair (diagnostic; logged, not reported)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work per workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size (counter calibration runs)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store HBM bytes per launch from two counter runs (no GPU needed)")
    ap.add_argument("--traffic-command", default="", help="the profiled command, stored with --record-traffic")
    args = ap.parse_args()

    if args.record_traffic:
        from workloads import configs
        wl = {"decode_grouped_kernel": configs.CONFIGS[args.config].name,
              "gemm_grouped_kernel": configs.CONFIGS[args.prefill_config].name}
        record_traffic(*args.record_traffic, args.copy_probe_mib or 512, wl, args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_wise_int4_amd import mnb
    from workloads import configs

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

    cfg = configs.CONFIGS[args.config]
    dec = run_workload(cfg, args.steps, args.warmup, not args.no_per_linear, torch, dev, args.launch_events)
    gbs = dec["bytes"] / (dec["ms"] * 1e-3) / 1e9
    # one launch per step: the kernel's algorithmic bytes per launch are the step's
    k_gbs = dec["bytes"] / (dec.get("launch_ms", dec["ms"]) * 1e-3) / 1e9
    decode_kernel = "decode_grouped_kernel" if cfg.m == 1 else "gemm_grouped_kernel"
    dec_traffic = stored_traffic(f"{decode_kernel}:{cfg.name}")

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
            "per_linear_ms_per_step": round(dec.get("per_linear_ms", float("nan")), 5),
            "per_linear_GBps": round(dec["bytes"] / (dec["per_linear_ms"] * 1e-3) / 1e9, 2)
            if "per_linear_ms" in dec else None,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": dec_traffic,
            "kernel": decode_kernel, "launch_us": round(dec.get("launch_ms", dec["ms"]) * 1e3, 2),
            "launch_timing": "timed region / steps (one launch per step, back to back)",
            "algorithmic_bytes_per_launch": dec["bytes"],
        },
    }

    if any(l.proj == "lm_head" for l in cfg.linears) and not args.no_next:
        result["lm_head_argmax"] = run_lm_head_argmax(cfg, args.steps, args.warmup, torch, dev)
        result["embedding_gather"] = run_embed_gather(cfg, args.steps, args.warmup, torch, dev)

    if args.prefill_config >= 0:
        pcfg = configs.CONFIGS[args.prefill_config]
        pre = run_workload(pcfg, max(5, args.steps // 10), max(2, args.warmup // 10), not args.no_per_linear,
                           torch, dev, args.launch_events)
        tf = pre["flops"] / (pre["ms"] * 1e-3) / 1e12
        k_tf = pre["flops"] / (pre.get("launch_ms", pre["ms"]) * 1e-3) / 1e12
        result["prefill"] = {
            "workload": pcfg.name, "M": pcfg.m, "linears": len(pcfg.linears), "value": round(tf, 2),
            "unit": "TFLOP/s", "ms_per_step": round(pre["ms"], 5), "schedule": "grouped",
            "launches_per_step": pre["launches_per_step"],
            "per_linear_TFLOPs": round(pre["flops"] / (pre["per_linear_ms"] * 1e-3) / 1e12, 2)
            if "per_linear_ms" in pre else None,
            "roofline": {"bound": "mfma", "achieved": round(k_tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(k_tf / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": stored_traffic(f"gemm_grouped_kernel:{pcfg.name}"),
                         "kernel": "gemm_grouped_kernel",
                         "launch_us": round(pre.get("launch_ms", pre["ms"]) * 1e3, 2),
                         "launch_timing": "timed region / steps (one launch per step, back to back)",
                         "algorithmic_flops_per_launch": pre["flops"]},
        }

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {cfg.name} (budget {args.cpu_budget:.0f}s)")
        cb = cpu_baseline(cfg, args.cpu_budget)
        result["cpu_baseline"] = {
            "value": round(cb["bytes"] / cb["seconds"] / 1e9, 4), "unit": "GB/s",
            "cores": cb["threads"], "kind": "oracle", "sample": cb["sample"],
        }
        if args.prefill_config >= 0:
            pcfg = configs.CONFIGS[args.prefill_config]
            log(f"[bench] cpu baseline: oracle on {pcfg.name}")
            pb = cpu_baseline(pcfg, args.cpu_budget)
            result["prefill"]["cpu_baseline"] = {
                "value": round(pb["flops"] / pb["seconds"] / 1e12, 5), "unit": "TFLOP/s",
                "cores": pb["threads"], "kind": "oracle", "sample": pb["sample"],
            }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
