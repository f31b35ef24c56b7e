"""The host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The host sources (descriptors and their flag entries, argument and limit checks,
dispatch, the pool share files and pages, the block's GEMM plans) are rebuilt with both
sanitizers and linked against the ordinary kernel objects; every host-side ABI test then
runs against that build in a child process with the sanitizer runtime preloaded.  Any
heap or stack overflow, use after free or undefined behaviour aborts the child.  CPU
only: no call reaches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "falcon_attention_kv_amd"))
import build as B  # noqa: E402


def test_host_paths_are_clean_under_asan_and_ubsan():
    try:
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if not all(os.path.exists(os.path.join(B.OUT_DIR, os.path.splitext(s)[0] + ".o"))
               for s in B.SOURCES if s.endswith(".hip")):
        pytest.skip("kernel objects missing: build the library first")
    lib = B.build_host_sanitized()
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_sanitized_runner.py"), lib],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "sanitized library mapped: True; plain library mapped: False" in out, out[-2000:]
