"""The host layer of the library (argument validation, path planning,
workspace layout -- all of ttq_api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: it is rebuilt with both, linked with the regular
kernel objects, and the whole C-ABI test file runs against it in a child
process with the ASan runtime preloaded.  Any sanitizer report fails the
test (halt_on_error; undefined behaviour does not recover).  No GPU is used:
those tests never launch a kernel."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_is_clean_under_host_sanitizers(tmp_path):
    from online_activation_aware_ttq_amd import build as B
    try:
        lib = B.build_host_sanitized(str(tmp_path))
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"sanitized build unavailable: {e}")
    # the library really is instrumented
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, TTQ_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x",
                          "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
