"""Builds libmtpdraft.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python mtp_draft_head_02_amd/build.py

hipcc cross-compiles without a GPU. No fast-math; f32 division and square
root correctly rounded (the quantizers' codes depend on it); FP contraction off;
packed-FP32 instruction selection disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmtpdraft.so")
SOURCES = ["sweep.hip", "quant.hip", "abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmtpdraft.so)")


def command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fno-fast-math", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wall",
        "-I", os.path.join(ROOT, "include"),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmtpdraft.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
