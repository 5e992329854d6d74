"""Builds the native libraries in-tree.

* libgpt2mi.so   - the HIP kernels and the C ABI (hipcc, gfx950 only).
* libgpt2synth.so - the seeded input generator's fill routines (gcc, OpenMP).

Run ``python -m gpt_pre_norm_amd.build``; ``__graft_entry__.build()`` calls it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gpt2mi.hip", "embed_ln.hip", "gemm.hip", "attention.hip", "generate.hip", "loss.hip"]
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: left to itself the compiler parked the
    # attention's accumulators in AGPRs and copied them back and forth every
    # key tile (96 v_accvgpr moves per tile per wave)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]

LIB = os.path.join(HERE, "libgpt2mi.so")
SYNTH_LIB = os.path.join(HERE, "libgpt2synth.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build_synth() -> str:
    _run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", SYNTH_LIB,
          os.path.join(HERE, "synth.c"), "-lm"])
    return SYNTH_LIB


def build_hip(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def build() -> None:
    build_synth()
    build_hip()


if __name__ == "__main__":
    build()
    print("built", LIB, SYNTH_LIB, file=sys.stderr)
