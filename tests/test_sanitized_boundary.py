"""The C-ABI boundary tests again, against the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (argument validation,
workspace and alias checks, planning, environment parsing).  Device code is
the regular build's; nothing here launches a kernel."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_tests_pass_under_asan_and_ubsan():
    from gemv_prefill_decode_amd import build as b
    if not os.path.isdir(b.BUILD_DIR) or not all(
            os.path.exists(os.path.join(b.BUILD_DIR, s + ".o")) for s in b.SOURCES):
        pytest.skip("regular build objects missing (run __graft_entry__.build())")
    try:
        san = b.build_sanitized()
        rt = b.asan_runtime()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    syms = subprocess.run(["nm", "-D", san], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "library is not instrumented"
    env = dict(os.environ, QMM_LIBRARY=san, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_boundary.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
