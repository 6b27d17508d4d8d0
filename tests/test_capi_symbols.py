"""The C-ABI library loads on a host without a GPU and exports every symbol include/kvattn.h declares."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(kvattn_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kvattn_plan", "kvattn_decode", "kvattn_plan_upload", "kvattn_plan_device_bytes",
                     "kvattn_forward", "kvattn_merge", "kvattn_plan_stats", "kvattn_plan_export",
                     "kvattn_decode_append", "kvattn_decode_streams", "kvattn_plan_update", "kvattn_expand_query_tokens",
                     "kvattn_plan_destroy", "kvattn_status_string", "kvattn_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    K = pytest.importorskip("decode_attention_prefix_amd.kvattn")
    out = subprocess.check_output(["nm", "-D", "--defined-only", K.LIB_PATH]).decode()
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(K.EXPORTED) <= exported


def test_header_compiles_as_c():
    src = '#include "kvattn.h"\nint main(void){kvattn_plan_options o; kvattn_plan_options_default(&o); return 0;}\n'
    tmp = os.path.join(ROOT, "_build")
    os.makedirs(tmp, exist_ok=True)
    cfile = os.path.join(tmp, "hdr_check.c")
    with open(cfile, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c", cfile,
                           "-o", os.path.join(tmp, "hdr_check.o")])


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: the binding, loaded where no libkvattn.so was built, refuses to import."""
    import shutil
    import sys
    shutil.copy(os.path.join(ROOT, "decode_attention_prefix_amd", "kvattn.py"), str(tmp_path / "kvattn.py"))
    env = {k: v for k, v in os.environ.items() if k != "KVATTN_LIBRARY"}
    r = subprocess.run([sys.executable, "-c", "import kvattn"], cwd=str(tmp_path), capture_output=True, text=True,
                       env=env)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libkvattn.so is not built" in r.stderr


def test_trace_hook_only_in_the_trace_build():
    """The per-task trace hook exists in the diagnostic build (_build/trace) and not in the library."""
    from decode_attention_prefix_amd import build as B

    def exported(path):
        out = subprocess.check_output(["nm", "-D", "--defined-only", path]).decode()
        return set(line.split()[-1] for line in out.splitlines() if line.strip())

    if not os.path.exists(B.LIB):
        pytest.skip("library not built")
    assert "kvattn_trace_set" not in exported(B.LIB)
    if os.path.exists(B.TRACE_LIB):
        assert "kvattn_trace_set" in exported(B.TRACE_LIB)
