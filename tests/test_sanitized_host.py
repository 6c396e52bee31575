"""The CPU tests once more under AddressSanitizer and UndefinedBehaviorSanitizer:
the float64 oracle and the host side of libpagedattn (argument checks, host
validators, block manager) built with -fsanitize=address,undefined, run in a
child pytest with the sanitizer runtime preloaded (tests/sanitize/
run_sanitized.py).  Any report aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))


def _have_toolchain():
    if not (shutil.which("gcc") and shutil.which("g++")):
        return False
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return os.path.isabs(asan) and os.path.exists(asan) and os.path.exists("/opt/rocm/include")


@pytest.mark.skipif(os.environ.get("PA_SANITIZED_RUN") == "1",
                    reason="this is the sanitized child run itself")
@pytest.mark.skipif(not _have_toolchain(), reason="gcc with libasan or the HIP headers missing")
def test_cpu_tests_clean_under_asan_and_ubsan():
    import run_sanitized
    libs = run_sanitized.build()
    r = run_sanitized.run_tests(libs)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
