"""Host-only C++ tests, built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (no HIP, no GPU): the argument validation layer,
and the attention launch plan (its invariants over a sweep of shapes, and the
plans the GPU tests and the benchmark are written against)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validate_under_sanitizers(tmp_path):
    exe = tmp_path / "test_validate"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-include", "string", "-I", os.path.join(ROOT, "long_context_self_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_cpp", "test_validate.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "OK (0 failures)" in res.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_launch_plan_under_sanitizers(tmp_path):
    exe = tmp_path / "test_launch_plan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "long_context_self_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_cpp", "test_launch_plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "OK (0 failures)" in res.stdout
