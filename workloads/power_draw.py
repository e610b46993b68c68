"""Board power and engine clocks while one workload's step runs back to back.

Context for the rooflines: the MFMA-bound prefill steps run at the board's
power limit, where the clock falls as the matrix pipes get busier, so a
kernel's MFMA busy fraction and its clock trade against each other.

    python -m workloads.power_draw --configs 1,3,4 --seconds 5 [--out FILE.md]

For each workload (an index into workloads.configs.CONFIGS) the grouped
plan's single launch runs back to back for about --seconds, with a host
synchronization every 200 launches, while a thread samples
`amd-smi metric -g 0 -p -c --json` (socket power and the engine clock of
each XCD). The samples of the 1.5 s before the loop give the idle figures;
those from 0.5 s after its start to 0.3 s before its end give the busy ones.
A measurement tool: nothing in the library or the tests runs it.
"""

import argparse
import json
import os
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def sample_loop(stop, out, period=0.2):
    while not stop.is_set():
        t = time.time()
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True,
                               text=True, timeout=5)
            out.append((t, r.stdout))
        except (OSError, subprocess.SubprocessError):
            pass
        time.sleep(period)


def parse(stdout):
    """(socket power in W, [engine clock of each XCD in MHz]) or None."""
    try:
        j = json.loads(stdout)
    except ValueError:
        return None
    if isinstance(j, dict):
        j = j.get("gpu_data", [j])
    g = j[0]
    try:
        power = float(g["power"]["socket_power"]["value"])
        clocks = [float(g["clock"][f"gfx_{i}"]["clk"]["value"]) for i in range(8) if f"gfx_{i}" in g["clock"]]
    except (KeyError, TypeError, ValueError):
        return None
    return power, clocks


def measure(ci, seconds, dev):
    import torch

    from block_wise_int4_amd import mnb, workload
    from workloads import configs

    cfg = configs.CONFIGS[ci]
    base = workload.build_config(cfg, dev).linears
    plan = workload.make_plan(cfg, base)
    step = lambda: mnb.mnb_gemm_grouped(plan)  # noqa: E731
    for _ in range(20):
        step()
    torch.cuda.synchronize()
    t = time.time()
    for _ in range(50):
        step()
    torch.cuda.synchronize()
    n = max(200, int(seconds / max((time.time() - t) / 50, 1e-6)))
    samples, stop = [], threading.Event()
    th = threading.Thread(target=sample_loop, args=(stop, samples))
    th.start()
    time.sleep(1.5)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    s.record()
    for i in range(n):
        step()
        if i % 200 == 199:
            torch.cuda.synchronize()
    e.record()
    torch.cuda.synchronize()
    t1 = time.time()
    stop.set()
    th.join()
    us = s.elapsed_time(e) / n * 1e3
    busy = [p for ts, out in samples if t0 + 0.5 <= ts <= t1 - 0.3 for p in [parse(out)] if p]
    idle = [p for ts, out in samples if ts < t0 for p in [parse(out)] if p]
    del plan, base
    torch.cuda.empty_cache()
    rec = {"workload": cfg.name, "launches": n, "us_per_launch": round(us, 2), "busy_samples": len(busy),
           "idle_samples": len(idle)}
    if busy:
        pw = [p for p, _ in busy]
        clk = [c for _, cs in busy for c in cs]
        rec.update(power_w_median=statistics.median(pw), power_w_min=min(pw), power_w_max=max(pw),
                   clock_mhz_median=statistics.median(clk), clock_mhz_min=min(clk), clock_mhz_max=max(clk))
    if idle:
        rec.update(idle_power_w_median=statistics.median([p for p, _ in idle]),
                   idle_clock_mhz_median=statistics.median([c for _, cs in idle for c in cs]))
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--configs", default="1,3,4")
    ap.add_argument("--seconds", type=float, default=5.0)
    ap.add_argument("--out", default=None, help="also write a markdown summary here")
    a = ap.parse_args()
    recs = []
    for ci in [int(c) for c in a.configs.split(",") if c]:
        rec = measure(ci, a.seconds, "cuda:0")
        print(json.dumps(rec), flush=True)
        recs.append(rec)
    if a.out:
        cmd = "python -m workloads.power_draw " + " ".join(sys.argv[1:])
        lines = ["# Board power and engine clocks under sustained launches", "",
                 "One MI355X, run from the repository root; `amd-smi` socket power and the engine clock of each "
                 "XCD, sampled about every 0.3 s while the workload's grouped step (one launch) runs back to back.",
                 "", "```", cmd, "```", "",
                 "| workload | us per launch | power (W): median (min-max) | clock (MHz): median (min-max) "
                 "| idle power (W) | idle clock (MHz) |", "|---|---:|---:|---:|---:|---:|"]
        for r in recs:
            lines.append(f"| {r['workload']} | {r['us_per_launch']} | {r.get('power_w_median')} "
                         f"({r.get('power_w_min')}-{r.get('power_w_max')}) | {r.get('clock_mhz_median')} "
                         f"({r.get('clock_mhz_min')}-{r.get('clock_mhz_max')}) | {r.get('idle_power_w_median')} "
                         f"| {r.get('idle_clock_mhz_median')} |")
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
