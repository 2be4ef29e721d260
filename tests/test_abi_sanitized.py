"""The C-ABI tests (tests/test_abi.py) against a host build of the C-ABI layer with
AddressSanitizer and UndefinedBehaviorSanitizer: lard_api.cpp compiled by g++ with
-fsanitize=address,undefined and linked with host stand-ins for the device launchers
(tests/sanitize/stub_launch.cpp, every launch fails).  Validation, sizing and launch
assembly run exactly as in liblard.so; any sanitizer report fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_relation_distillation_amd", "csrc")


def test_abi_tests_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    libasan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan not available")
    lib = tmp_path / "liblard_sanitized.so"
    cmd = [gxx, "-std=c++20", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "lard_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.update(LARD_LIBRARY=str(lib), LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out
