"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, and
the HBM-traffic bookkeeping (counter calibration against a plain device copy,
bytes per launch, records tied to the kernel sources they were taken on)."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_record_traffic_calibrates_each_counter_on_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    probe_mib = 512
    copy_kib = probe_mib * 1024
    # FETCH_SIZE reads half of the copied bytes, WRITE_SIZE all of them; two
    # launches of each kernel are averaged; a smaller copy is not the probe
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2), ("__amd_rocclr_copyBuffer", 10.0),
                                       ("mnb::decode_grouped_kernel<...>", 1000.0),
                                       ("mnb::decode_grouped_kernel<...>", 1200.0),
                                       ("void mnb::gemm_grouped_kernel<13, 2>", 4000.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib), ("mnb::decode_grouped_kernel<...>", 8.0),
                                       ("mnb::decode_grouped_kernel<...>", 12.0),
                                       ("void mnb::gemm_grouped_kernel<13, 2>", 300.0)])
    workloads = {"decode_grouped_kernel": "decode-a", "gemm_grouped_kernel": "prefill-b"}
    bench.record_traffic(str(fetch), str(write), probe_mib, workloads, "the command")
    data = json.load(open(tmp_path / "traffic.json"))
    dec = data["decode_grouped_kernel:decode-a"]
    assert dec["fetch_factor"] == 2.0 and dec["write_factor"] == 1.0
    assert dec["bytes_per_launch"] == round(1100.0 * 1024 * 2 + 10.0 * 1024)
    assert dec["source_sha"] == bench.kernel_source_sha("decode_grouped_kernel")
    assert dec["command"] == "the command"
    gemm = data["gemm_grouped_kernel:prefill-b"]
    assert gemm["bytes_per_launch"] == round(4000.0 * 1024 * 2 + 300.0 * 1024)
    assert bench.stored_traffic("decode_grouped_kernel:decode-a") == dec["bytes_per_launch"]


def test_record_traffic_needs_the_copy_probe(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("mnb::decode_grouped_kernel", 1.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1.0)])
    with pytest.raises(SystemExit):
        bench.record_traffic(str(fetch), str(write), 512, {"decode_grouped_kernel": "w"}, "")


def test_traffic_taken_on_other_sources_is_ignored(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    sha = bench.kernel_source_sha("gemm_grouped_kernel")
    assert len(sha) == 16 and int(sha, 16) >= 0
    json.dump({"gemm_grouped_kernel:w": {"bytes_per_launch": 7, "source_sha": sha},
               "gemm_grouped_kernel:old": {"bytes_per_launch": 9, "source_sha": "0" * 16}}, open(path, "w"))
    assert bench.stored_traffic("gemm_grouped_kernel:w") == 7
    assert bench.stored_traffic("gemm_grouped_kernel:old") is None
    assert bench.stored_traffic("gemm_grouped_kernel:absent") is None


def test_committed_traffic_records_name_their_sources():
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert data
    for key, rec in data.items():
        kernel = key.split(":")[0]
        assert kernel in bench.KERNEL_SOURCES
        assert rec["bytes_per_launch"] > 0 and rec["fetch_factor"] > 0 and rec["write_factor"] > 0
        assert len(rec["source_sha"]) == 16 and "rocprofv3 --pmc" in rec["command"]


def test_mfma_counters_attach_to_prefill_rooflines(tmp_path, monkeypatch):
    """A counter record of the current kernel source adds the busy fraction
    and the rate against the dense peak at the measured clock to an
    MFMA-bound leg; one taken on other sources, or a decode leg, adds none."""
    from workloads import configs

    path = tmp_path / "mfma.json"
    monkeypatch.setattr(bench, "MFMA_COUNTERS_FILE", str(path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.json"))
    sha = bench.kernel_source_sha("gemm_grouped_kernel")
    pre = configs.CONFIGS[3]
    json.dump({f"gemm_grouped_kernel:{pre.name}": {"source_sha": sha, "mfma_busy_fraction": 0.5, "clock_ghz": 2.0}},
              open(path, "w"))
    res = {"ms": 1.0, "bytes": 10**9, "flops": 10**12, "replicas": 2, "launches_per_step": 1,
           "first_launch_ms": 2.0, "steps": 40, "warmup": 20}
    roof = bench.leg_record(pre, res, "gemm_grouped_kernel")["roofline"]
    c = roof["counters"]
    assert c["mfma_busy_fraction"] == 0.5 and c["clock_ghz"] == 2.0
    assert c["peak_at_clock"] == round(256 * 4096 * 2.0 / 1e3, 1)  # 2097.2 TFLOP/s
    assert c["frac_at_clock"] == round(roof["achieved"] / c["peak_at_clock"], 4)
    assert roof["frac"] == round(roof["achieved"] / 2500.0, 4)
    json.dump({f"gemm_grouped_kernel:{pre.name}": {"source_sha": "0" * 16, "mfma_busy_fraction": 0.5,
                                                    "clock_ghz": 2.0}}, open(path, "w"))
    assert "counters" not in bench.leg_record(pre, res, "gemm_grouped_kernel")["roofline"]
    dec = configs.CONFIGS[1]
    assert "counters" not in bench.leg_record(dec, res, "decode_grouped_kernel")["roofline"]


def test_committed_mfma_counter_records_name_their_sources():
    data = json.load(open(os.path.join(ROOT, "profiles", "mfma_counters.json")))
    assert data
    for key, rec in data.items():
        assert key.split(":")[0] == "gemm_grouped_kernel"
        assert 0 < rec["mfma_busy_fraction"] < 1 and 1.0 < rec["clock_ghz"] < 2.5
        assert len(rec["source_sha"]) == 16 and "rocprofv3 --pmc" in rec["command"]
