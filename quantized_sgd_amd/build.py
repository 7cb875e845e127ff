"""Builds libqsgd.so (gfx950) in-tree with hipcc.

Flags: -ffp-contract=off keeps every floating-point expression one IEEE op at a
time (the quantizer's decisions must be reproducible bit for bit); packed fp32
instructions are disabled; denormals are kept (no flush-to-zero).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqsgd.so")
SOURCES = [os.path.join(HERE, "csrc", "qsgd_api.hip")]
ARCH = os.environ.get("QSGD_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str = LIB, extra=()):
    return [
        "/opt/rocm/bin/hipcc", "-O3", "-std=c++17", f"--offload-arch={ARCH}",
        "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
        "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wshadow", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *extra, "-o", out, *SOURCES,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
