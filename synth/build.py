"""Builds, for gfx950 and in-tree, synth/libzsynth.so (the device-side input
generator) and synth/libzprobe.so (the streaming probes that give the bench its
practical HBM ceilings)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libzsynth.so")
PROBE_LIB = os.path.join(HERE, "libzprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, os.path.join(HERE, "csrc", src), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _hipcc("synth_gen.hip", LIB, verbose)
    _hipcc("stream_probe.hip", PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
