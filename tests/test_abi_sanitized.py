"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

build_sanitized() compiles api.hip, the host code behind every entry point (argument checks,
sizes, workspace and flag rules, the library's error string), with both sanitizers on its host
pass; the kernels are built as usual and none is launched here. tests/test_abi.py, which includes
the plain C consumer, then runs in a child Python process that loads that library with the
sanitizer runtime preloaded (Python itself is not instrumented). Any report aborts the child and
fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_under_sanitizers(tmp_path):
    from context_attention_dits_amd import build
    try:
        rt = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized(str(tmp_path / "sanitized"))
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout and "__ubsan_handle_" in nm.stdout, "library not instrumented"
    preload = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, CP_ATTN_LIBRARY=lib, LD_PRELOAD=rt + (":" + preload if preload else ""),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
