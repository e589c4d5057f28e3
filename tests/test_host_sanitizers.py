"""The C ABI's host-side argument validation (q8_validate.h, pure C++) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and run through every check function's
accepted boundary values and error paths (tests/host/validate_sanitized.cpp).  CPU only:
no HIP code is compiled here."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "validate_sanitized.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_sanitized")
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *flags,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "block_quantized_weight_linear_amd", "csrc"),
           SRC, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    # a preloaded library of the environment may come before the ASan runtime
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all cases as expected" in run.stdout
