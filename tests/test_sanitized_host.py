"""The host code of libpab.so (argument validation, the planner, the
dispatcher's checks, the launchers' bookkeeping) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

``python -m reuse_pab_plan_amd.build --sanitize`` builds libpab_san.so (host
passes only; device code unchanged).  When that build exists and is newer
than every source, this test runs the library-facing CPU tests in a child
process against it with the ASan runtime preloaded; any sanitizer report
aborts the child and fails the test.  Without a current build it is skipped.
"""

import glob
import os
import subprocess
import sys

import pytest

from reuse_pab_plan_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = build.LIB_SAN


def _current():
    if not os.path.exists(SAN):
        return False
    t = os.path.getmtime(SAN)
    srcs = glob.glob(os.path.join(build.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return all(os.path.getmtime(s) <= t for s in srcs)


@pytest.mark.skipif(not _current(), reason="no current libpab_san.so (build with --sanitize)")
def test_library_facing_cpu_tests_under_sanitizers():
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), PAB_LIB=SAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_abi_cpu.py", "test_oracle_calibration.py", "test_synth_cpu.py",
              "test_oracle_schedule.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider", *tests],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(res.stdout[-2000:], res.stderr[-2000:])
    assert res.returncode == 0
    assert "passed" in res.stdout and "AddressSanitizer" not in res.stderr
