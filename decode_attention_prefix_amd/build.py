"""Build libkvattn.so in-tree: host planner (g++), HIP runtime glue and gfx950 kernels (hipcc).

Usage: python -m decode_attention_prefix_amd.build   (or build() from Python)
Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvattn.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    print("+ " + " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose_isa: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    plan_o = os.path.join(BUILD, "kvattn_plan.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
          os.path.join(CSRC, "kvattn_plan.cpp"), "-o", plan_o])
    objs.append(plan_o)
    rt_o = os.path.join(BUILD, "kvattn_runtime.o")
    _run([HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", ROCM_INCLUDE, "-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c",
          os.path.join(CSRC, "kvattn_runtime.cpp"), "-o", rt_o])
    objs.append(rt_o)
    k_o = os.path.join(BUILD, "kvattn_kernels.o")
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, *NO_PACKED_FP32, "-c",
           os.path.join(CSRC, "kvattn_kernels.hip"), "-o", k_o]
    if verbose_isa:
        cmd += ["-save-temps=obj"]
    _run(cmd)
    objs.append(k_o)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose_isa="--isa" in sys.argv)
