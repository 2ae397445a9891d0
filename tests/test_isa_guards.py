"""The device code as built (CPU only: hipcc cross-compiles to gfx950 assembly):
every HIP source of the library, of the input generator and of the streaming
probes, compiled with the flags its build script uses, holds no packed-fp32
arithmetic -- the builds leave that feature out of code generation, and this
test keeps it out."""
import importlib.util
import os
import re
import subprocess

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PACKED = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _load(rel):
    spec = importlib.util.spec_from_file_location("b_" + rel.replace("/", "_")[:-3],
                                                  os.path.join(ROOT, rel))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _device_asm(src, flags, includes, out):
    cmd = [HIPCC, *[f for f in flags if f not in ("-shared", "-fPIC")], "--cuda-device-only",
           "-S", *sum((["-I", i] for i in includes), []), src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return open(out).read()


@pytest.mark.slow
def test_no_packed_fp32_in_any_device_code(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    zb = _load("zero_sharded_mixed_bucketed_amd/_build.py")
    sb = _load("synth/build.py")
    cases = [(s, zb.HIP_FLAGS, [os.path.join(ROOT, "include"), os.path.dirname(s)])
             for s in zb.sources()]
    for name in ("synth_gen.hip", "stream_probe.hip"):
        cases.append((os.path.join(ROOT, "synth", "csrc", name), sb.FLAGS, []))
    for i, (src, flags, inc) in enumerate(cases):
        asm = _device_asm(src, flags, inc, str(tmp_path / f"k{i}.s"))
        if "__global__" in open(src).read():                     # it holds kernels
            assert ".amdhsa_kernel" in asm and "v_" in asm, src
        hits = sorted(set(m.group(0) for m in PACKED.finditer(asm)))
        assert not hits, (os.path.basename(src), hits)
