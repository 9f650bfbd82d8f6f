"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The library's host side (include/specverify.h entry points, argument checks
  and the launch plan in sv_api.cpp), linked against launchers that only
  record their parameters: every check answers before a launch, and each
  plan -- the capped early exit above all -- keeps its workspace regions
  inside the caller's buffer.
* The CPU oracle (oracle/svo.c) on small seeded cases of every entry point.

Both are compiled with gcc/g++ as host-only programs (no HIP code), each in a
build of its own: the oracle and the library share no code.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} is not installed")


def _run(cmd, exe, tmp_path):
    subprocess.run(cmd, check=True, cwd=tmp_path)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    return r.stdout


def test_host_plan_under_sanitizers(tmp_path):
    _need("g++")
    exe = tmp_path / "host_plan_check"
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "draft_token_verification_10_amd", "csrc"),
           os.path.join(ROOT, "draft_token_verification_10_amd", "csrc", "sv_api.cpp"),
           os.path.join(ROOT, "tests", "c", "host_plan_check.cpp"), "-o", str(exe)]
    assert "host plan checks ok" in _run(cmd, exe, tmp_path)


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c99", *SAN, "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "svo.c"), os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
           "-o", str(exe), "-lm"]
    assert "oracle sanitizer checks ok" in _run(cmd, exe, tmp_path)
