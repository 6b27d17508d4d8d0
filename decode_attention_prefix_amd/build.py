"""Build libkvattn.so in-tree: host planner (g++), HIP runtime glue and gfx950 kernels (hipcc).

Usage: python -m decode_attention_prefix_amd.build [--sanitize]   (or build() from Python)
Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (-Xclang -target-feature -Xclang -packed-fp32-ops).

build() also makes _build/trace/libkvattn.so, a diagnostic variant whose
forward kernel writes per-task trace records (compiled with
-DKVATTN_TASK_TRACE; task_trace.py loads it).  The library itself carries no
trace code: without the macro the kernels compile to the same instructions.

build(sanitize=True) makes a checking variant for host tests only,
_build/san/libkvattn.so: the host planner (the part that indexes caller
tables, trees and lengths) is compiled by g++ with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts), linked by g++ with the
unchanged runtime and kernel objects.  Load it with KVATTN_LIBRARY pointing at
it and libasan / libubsan preloaded (tests/test_sanitized_planner.py does).
It never runs on a GPU: the sanitizers cover host code only.
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


TRACE_DIR = os.path.join(BUILD, "trace")
TRACE_LIB = os.path.join(TRACE_DIR, "libkvattn.so")
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libkvattn.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_sanitized() -> str:
    """The host planner under ASan + UBSan, linked with the regular runtime and kernel objects
    (rebuilt first when missing or older than their sources)."""
    objs = [os.path.join(BUILD, n) for n in ("kvattn_runtime.o", "kvattn_kernels.o")]
    newest_src = max(os.path.getmtime(os.path.join(d, f)) for d in (CSRC, INCLUDE) for f in os.listdir(d))
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest_src for o in objs):
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    plan_o = os.path.join(SAN_DIR, "kvattn_plan_san.o")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *SAN_FLAGS, "-I", INCLUDE, "-c",
          os.path.join(CSRC, "kvattn_plan.cpp"), "-o", plan_o])
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    tmp = SAN_LIB + ".tmp%d" % os.getpid()
    _run(["g++", "-shared", *SAN_FLAGS, plan_o, os.path.join(BUILD, "kvattn_runtime.o"),
          os.path.join(BUILD, "kvattn_kernels.o"), "-L", rocm_lib, "-Wl,-rpath," + rocm_lib, "-lamdhip64",
          "-o", tmp])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build_trace() -> str:
    """The per-task trace variant: kernels with -DKVATTN_TASK_TRACE, linked with the regular
    planner and runtime objects (built by build())."""
    os.makedirs(TRACE_DIR, exist_ok=True)
    k_o = os.path.join(TRACE_DIR, "kvattn_kernels_trace.o")
    _run([HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-DKVATTN_TASK_TRACE", "-I", INCLUDE,
          *NO_PACKED_FP32, "-c", os.path.join(CSRC, "kvattn_kernels.hip"), "-o", k_o])
    tmp = TRACE_LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, os.path.join(BUILD, "kvattn_plan.o"),
          os.path.join(BUILD, "kvattn_runtime.o"), k_o, "-o", tmp])
    os.replace(tmp, TRACE_LIB)
    return TRACE_LIB


def build(verbose_isa: bool = False, sanitize: bool = False, trace: bool = True) -> str:
    if sanitize:
        return build_sanitized()
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
    if trace:
        build_trace()
    return LIB


if __name__ == "__main__":
    build(verbose_isa="--isa" in sys.argv, sanitize="--sanitize" in sys.argv)
