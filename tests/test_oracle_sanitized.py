"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The pin suite (tests/test_oracle_pins.py) is re-run in a child process against
liboracle_gdn_san.so, built from the same source with -fsanitize=address,undefined
and -fno-sanitize-recover, with the sanitizer runtimes preloaded. Any invalid
access, leak-free-use error or undefined behaviour in the oracle aborts the child
and fails this test. Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_pass_under_asan_and_ubsan():
    from oracle import build
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = build.build(sanitize=True)
    env = dict(os.environ, GDN_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in res.stdout
