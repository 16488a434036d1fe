"""Build libgpt2_mi355x.so (gfx950 only) next to this file.

    python -m scratch_transformer_lm_amd.build [-v]

Each csrc/*.hip file is compiled to an object under _build/ in parallel, then all are
linked into one shared library.  Packed-FP32 instruction selection is switched off for
device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgpt2_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = []
    procs = []
    jobs = jobs or min(8, os.cpu_count() or 4)
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        while len([p for p, _ in procs if p.poll() is None]) >= jobs:
            procs[[i for i, (p, _) in enumerate(procs) if p.poll() is None][0]][0].wait()
    errors = []
    for p, src in procs:
        _, err = p.communicate()
        msgs = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if p.returncode != 0:
            errors.append(f"{src}:\n{err}")
        elif msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    if errors:
        raise RuntimeError("HIP build failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
