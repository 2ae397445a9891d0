"""The kernels' indexing, checked on the CPU from their own source.

The reduce's and the stage-3 gather's index plans live in headers that the HIP
kernels and these checks both compile (csrc/reduce_plan.h, csrc/gather_plan.h).
Each check is built with g++ and walks every thread group (reduce) or every
workgroup of every launch (gather) as the kernel would, against the definition
of the operation:

* tests/native/reduce_plan_check.cpp -- every owned column reduced exactly once,
  outputs inside the shard, full groups inside the owned columns with aligned,
  in-bounds row loads and aligned stores; the launches of the 7.5B (ranks 0, 1,
  63), 13B and 100B workloads at the advised stride, and 20,000 random shapes
  column by column;
* tests/native/gather_plan_check.cpp -- the pieces tile the range in order, every
  workgroup of a piece hit once, aligned in-bounds accesses, every element
  written once on small cases; the device test cases, every layer of the 7.5B
  and 100B stacks, the top of the 64-bit range and 3,000 random shapes.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def _build_and_run(tmp_path, name, expect):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = tmp_path / name
    src = os.path.join(ROOT, "tests", "native", f"{name}.cpp")
    inc = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd", "csrc")
    r = subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror",
                        "-Wno-unknown-pragmas", "-I", inc, src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert expect in r.stdout


def test_reduce_plan_covers_every_owned_column_once(tmp_path):
    _build_and_run(tmp_path, "reduce_plan_check", "reduce plan check ok")


def test_gather_plan_covers_every_element_once(tmp_path):
    _build_and_run(tmp_path, "gather_plan_check", "gather plan check ok")
