"""The C ABI's host logic built for the CPU under AddressSanitizer and
UndefinedBehaviorSanitizer: argument validation (csrc/validate.h) and the
decode split plan and workspace layout (csrc/decode_plan.h), the same headers
the library compiles. tests/host/validate_check.cpp drives them over every
error path, the workloads' shapes and 200,000 pseudo-random size combinations
(including sizes far past the limits) and checks the plan invariants; any
sanitizer report is fatal."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "validate_check.cpp")


def test_validation_and_plan_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "validate_check")
    build = [cxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             SRC, "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: other preloaded libraries may come before the
    # sanitizer runtime in the process; the checks do not depend on the order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok:" in r.stdout
