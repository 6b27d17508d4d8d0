"""Structure of the compiled forward kernels (CPU; needs hipcc).

The persistent forward kernel's loops hold workgroup barriers.  If the
compiler turned a lane-divergent branch into an exec-masked loop (lanes of
one wave leaving the loop at different iterations) around a barrier, waves
would stop meeting at the barrier and the kernel would hang.  Its control
flow is kept wave-uniform on purpose; this test reads the gfx950 assembly the
compiler emits for every forward instantiation and checks that no loop whose
exit is taken per lane holds an s_barrier.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_prefix_amd", "csrc", "kvattn_kernels.hip")


def _assembly(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.dirname(SRC), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "--cuda-device-only", "-S", SRC, "-o", str(out)], stderr=subprocess.DEVNULL)
    return out.read_text().split("\n")


def _blocks(lines):
    """Basic blocks of the forward kernels: (innermost loop header or None, instruction lines)."""
    blocks, cur, in_fwd = [], None, False
    for line in lines:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            in_fwd = "fwd_kernel" in m.group(1)
            cur = None
            continue
        if not in_fwd:
            continue
        if line.startswith(".LBB") or line.startswith("; %bb."):
            ann = line.split(";", 1)[1] if ";" in line[1:] else ""
            name = line.split(":")[0][2:] if line.startswith(".LBB") else None
            hdr = re.search(r"Header=(BB\S+)", ann)
            loop = name if ("Loop Header" in ann and name) else (hdr.group(1) if hdr else None)
            cur = {"loop": loop, "lines": []}
            blocks.append(cur)
        elif cur is not None:
            cur["lines"].append(line)
    return blocks


def test_no_barrier_in_lane_divergent_loop(tmp_path):
    lines = _assembly(tmp_path)
    assert any("fwd_kernel" in l for l in lines)
    loops = {}
    for b in _blocks(lines):
        if b["loop"] is None:
            continue
        d = loops.setdefault(b["loop"], [False, False])
        d[0] |= any("s_andn2_b64 exec, exec" in x or "s_cbranch_execnz" in x for x in b["lines"])
        d[1] |= any("s_barrier" in x for x in b["lines"])
    bad = [k for k, (divergent_exit, barrier) in loops.items() if divergent_exit and barrier]
    assert not bad, "exec-masked loops holding a barrier: %s" % bad
