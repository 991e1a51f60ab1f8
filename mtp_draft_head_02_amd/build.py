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
# Translation units, compiled in parallel, then linked. The sweep kernels are
# templates in csrc/sweep_impl.h; each weight format's instantiations sit in a
# unit of their own (the largest units dominate the build time).
SOURCES = ["lm_bf16.hip", "lm_fp8.hip", "lm_nvfp4.hip", "mfma_bf16.hip", "mfma_fp8.hip", "mfma_nvfp4.hip",
           "combine_bf16.hip", "combine_fp8.hip", "combine_nvfp4.hip", "combine_mfma.hip", "sweep.hip", "scratch.hip", "quant.hip", "stream_probe.hip",
           "abi.cpp"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fno-fast-math", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wall"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmtpdraft.so)")


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
            os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def build(verbose: bool = False, out: str = LIB, jobs: int | None = None) -> str:
    """Compile every unit (in parallel) into a temporary directory and link."""
    import concurrent.futures
    import tempfile

    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="mtpdraft_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.splitext(src)[0] + ".o") for src in SOURCES]

        def one(i):
            cmd = compile_command(SOURCES[i], objs[i])
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(one, range(len(SOURCES))))
        for src, r in zip(SOURCES, results):
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed compiling {src}")
        tmp = out + ".tmp"
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libmtpdraft.so")
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
