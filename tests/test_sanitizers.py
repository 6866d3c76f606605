"""The CPU test-suite once more under AddressSanitizer and UndefinedBehaviorSanitizer.

The host code of libdlfusion (argument validation of every entry point, the BN fold, the fusion
pass, the FFN packing and workspace sizing, the tuning switches) and the oracle's C code run
instrumented (sanitize_build.py); a child Python process preloads clang's ASan runtime and runs
the CPU test files that exercise them.  Any sanitizer report ends the child with an error.
No GPU is touched: the host tests reject every device call before a HIP call.
"""
import os
import subprocess
import sys

import pytest

import sanitize_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = ["tests/test_host_lib.py", "tests/test_fusion_pass.py", "tests/test_fallback.py",
         "tests/test_oracle_pins.py", "tests/test_fusion_oracle.py", "tests/test_parity_readings.py"]


@pytest.mark.slow
def test_cpu_suite_under_asan_and_ubsan():
    rt = sanitize_build.asan_runtime()
    if rt is None or not os.path.exists(sanitize_build.HIPCC):
        pytest.skip("no clang ASan runtime or hipcc here")
    lib = sanitize_build.build_library()
    orc = sanitize_build.build_oracle()
    env = dict(os.environ, LD_PRELOAD=rt, DLF_LIBRARY=lib, ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu and not slow", *FILES],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    report = (r.stdout[-6000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
    assert "runtime error" not in report and "ERROR: AddressSanitizer" not in report, report
