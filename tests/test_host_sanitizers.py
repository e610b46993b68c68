"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only): every source is rebuilt with both sanitizers on its
host side (device code is built as usual and never runs), linked with the
plain-C check program tests/host/abi_host_check.c, and run. The program exercises
argument validation of every entry point, packed sizes, and grouped plans
(written, re-read and corrupted on the host); none of its calls reaches a
GPU."""

import os
import shutil
import subprocess

import pytest

from block_wise_int4_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the library")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    cc = B.hipcc()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        procs.append(subprocess.Popen([cc, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    drv = str(tmp_path / "abi_host_check.o")
    procs.append(subprocess.Popen([cc, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-x", "c", "-c",
                                   os.path.join(ROOT, "tests", "host", "abi_host_check.c"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([cc, *SAN, f"--offload-arch={B.ARCH}", *objs, drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi host checks passed" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
