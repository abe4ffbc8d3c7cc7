"""Compile the HIP library ``libnf4.so`` for gfx950, in-tree.

hipcc cross-compiles without a GPU.  Flags: no fast-math and no FMA
contraction (the codec's fp32 steps are specified as separately rounded
operations), packed fp32 instructions off, fp32 denormals kept (the default).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libnf4.so")
CPU_LIB_PATH = os.path.join(PKG, "libnf4cpu.so")
CPU_SOURCES = [os.path.join("cpu", "nf4_cpu.cpp")]
SOURCES = ["k_codec.hip", "k_select.hip", "k_gemm.hip", "k_variants.hip", "nf4_scratch.hip",
           "nf4_api.cpp"]
ARCH = os.environ.get("NF4_OFFLOAD_ARCH", "gfx950")


def command(out: str = LIB_PATH) -> list:
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def cpu_command(out: str = CPU_LIB_PATH) -> list:
    """The host-CPU pass (OpenMP, AVX2 baseline with an AVX-512 tile path chosen at run time,
    no FMA contraction)."""
    return ["g++", "-O3", "-march=x86-64-v3", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-o", out, *[os.path.join(PKG, s) for s in CPU_SOURCES]]


def build_cpu(verbose: bool = False) -> str:
    tmp = CPU_LIB_PATH + ".tmp"
    cmd = cpu_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, CPU_LIB_PATH)
    return CPU_LIB_PATH


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_cpu(verbose=True))
