"""The host side of libpingala (C ABI validation, the reference encoder,
tables, per-thread errors) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU: a driver program
(tests/sanitize/host_driver.cpp) over pg_api.cpp and pg_host.cpp, with the
device launchers replaced by stubs that refuse (tests/sanitize/device_stubs.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "qgemv_amd", "csrc")
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-pthread",
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"),
           os.path.join(csrc, "pg_api.cpp"), os.path.join(csrc, "pg_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
