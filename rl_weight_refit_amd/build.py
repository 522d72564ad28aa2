"""Build the relayout library (libreshard.so) for gfx950 with hipcc.

Usage: python -m rl_weight_refit_amd.build   (or build() from Python).
The library lands next to this file, in-tree, so that it travels with the
source tree; nothing is installed.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libreshard.so")

SOURCES = ["kernels.hip", "planner.cpp", "capi.cpp"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def command(out=LIB, extra=()):
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # packed fp32 ops stay off: the compiler must not emit them.
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC]
    cmd += list(extra)
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out]
    return cmd


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(out=tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
