"""Build libmnb.so (the HIP library behind include/mnb.h) for gfx950, in-tree.

    python -m block_wise_int4_amd.build          # or build() from Python

Each call recompiles every source; the result lands next to this file.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmnb.so")
SOURCES = ("mnb_api.hip", "mnb_aux.hip", "mnb_gemv.hip", "mnb_gemm.hip", "mnb_embed.hip", "mnb_int8.hip")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions (v_pk_fma_f32 and friends) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE semantics: no contraction of separate multiplies and adds, no
    # denormal flushing; fused multiply-adds are written explicitly
    "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def build(verbose=False, jobs=None, out=None, defines=()):
    """Compile every source for gfx950 and link libmnb.so in place (or at
    `out`, with extra -D `defines`, for tuning experiments)."""
    objdir = os.path.join(HERE, "_build") if out is None else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, cmd, pr in procs:
        text, _ = pr.communicate()
        # the host pass does not know the packed-fp32 feature and says so
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if pr.returncode != 0:
            failed.append((src, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{o}" for s, o in failed))
    lib = LIB if out is None else out
    tmp = lib + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
