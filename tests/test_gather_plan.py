"""The stage-3 gather's indexing, checked on the CPU: tests/native/gather_plan_check.cpp
is built with g++ from the same gather_plan.h the kernel compiles (the launch
plan and each workgroup's piece recovery), and checks exact coverage, bounds and
access alignment against the definition of the gather over the device test
cases, every layer of the 7.5B and 100B stacks, the top of the 64-bit range and
3,000 random shapes."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def test_gather_plan_covers_every_element_once(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = tmp_path / "gather_plan_check"
    src = os.path.join(ROOT, "tests", "native", "gather_plan_check.cpp")
    inc = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd", "csrc")
    r = subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror",
                        "-Wno-unknown-pragmas", "-I", inc, src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "gather plan check ok" in r.stdout
