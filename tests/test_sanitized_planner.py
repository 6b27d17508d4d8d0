"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer (CPU; no GPU).

The planner indexes caller block tables, prefix trees and lengths (tree
derivation and adoption, packing, splitting, descriptor serialisation, plan
updates, new-token slot checks).  This builds the library with the planner
compiled by g++ -fsanitize=address,undefined (every report aborts) and runs
the planner test files against it in a child process -- the random forests,
bad-tree and bad-id fuzz, the update walks and the multi-token and new-token
plans included.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLANNER_TESTS = ["tests/test_plan.py", "tests/test_plan_update.py", "tests/test_multi_token.py",
                 "tests/test_new_token.py"]


def _runtime(name):
    path = subprocess.check_output(["gcc", "-print-file-name=" + name]).decode().strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_planner_tests_pass_under_asan_and_ubsan():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    sys.path.insert(0, ROOT)
    from decode_attention_prefix_amd import build as B
    lib = B.build_sanitized()
    # the planner in this build is instrumented (its loads and stores call the ASan runtime)
    syms = subprocess.check_output(["nm", "-D", "--undefined-only", lib]).decode()
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    preload = [asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env.update(LD_PRELOAD=":".join(preload), KVATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *PLANNER_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout
