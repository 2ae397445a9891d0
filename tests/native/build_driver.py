"""Builds tests/native/build/abi_gpu_driver: the plain C consumer of libzero
(host C compiled with gcc against include/zero.h and the HIP runtime API,
linked to the in-tree libzero.so).  Test infrastructure."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd")
EXE = os.path.join(HERE, "build", "abi_gpu_driver")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "abi_gpu_driver.c"), "-o", tmp,
           "-L", PKG, "-lzero", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../../zero_sharded_mixed_bucketed_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed building abi_gpu_driver")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
