"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no device call): tests/native/abi_host_check.cpp is linked with the
library sources, with the sanitizers on the host side of the compilation only,
and must run clean."""
import os
import subprocess

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.slow
def test_abi_host_paths_clean_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    csrc = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    exe = str(tmp_path / "abi_host_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-x", "hip", os.path.join(ROOT, "tests", "native", "abi_host_check.cpp"),
           *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host check ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.slow
def test_abi_host_paths_clean_under_tsan_from_many_threads(tmp_path):
    """The host paths called from eight threads at once, under ThreadSanitizer."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    csrc = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    exe = str(tmp_path / "abi_thread_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=thread",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-x", "hip", os.path.join(ROOT, "tests", "native", "abi_thread_check.cpp"),
           *srcs, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi thread check ok" in r.stdout
    assert "ThreadSanitizer" not in r.stderr, r.stderr
