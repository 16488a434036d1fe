"""Build the CPU oracle (test infrastructure): one C file, two precisions.

    python oracle/build.py          # writes oracle/liboracle_f64.so and oracle/liboracle_f32.so

Plain gcc, -O3 with OpenMP and strict IEEE arithmetic (no fast-math, no FMA
contraction), for a generic x86-64-v3 host so the same build runs on any AVX2 machine.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.c")
FLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
         "-fPIC", "-shared", "-fvisibility=hidden", "-std=c11", "-Wall", "-Wextra",
         "-Wno-unused-parameter"]
TARGETS = {"f64": [], "f32": ["-DORACLE_REAL_FLOAT"]}


def lib_path(precision: str) -> str:
    return os.path.join(HERE, f"liboracle_{precision}.so")


def build_native(precision: str = "f32", verbose: bool = False) -> str:
    """The same source built for the host it runs on (-march=native instead of the
    portable x86-64-v3), as liboracle_<precision>_native.so: the benchmark's CPU
    baseline times this build on the machine that runs the GPU."""
    out = lib_path(precision + "_native")
    flags = [f for f in FLAGS if not f.startswith("-march=")] + ["-march=native"]
    cmd = ["gcc", *flags, *TARGETS[precision], SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> None:
    procs = []
    for prec, extra in TARGETS.items():
        out = lib_path(prec)
        cmd = ["gcc", *FLAGS, *extra, SRC, "-o", out + ".tmp", "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), out))
    for p, out in procs:
        if p.wait() != 0:
            raise RuntimeError(f"oracle build failed: {out}")
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
