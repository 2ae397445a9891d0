"""bench.py end to end on the tiny workload, as a child process: it prints one
JSON line with the contract's fields, a roofline object for an HBM-bound kernel,
and a sampled self-check that is bit-exact against the oracle.  Five timed steps
on a workload of three: the live state takes t = 1..3 and the last two timed
steps, like the warm-up, run on the scratch copy, so the checked trajectory is
the workload's own."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def test_bench_tiny_prints_one_contract_line():
    need_gpu()
    print("bench smoke: tiny-zero2", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny-zero2",
                        "--steps", "5", "--warmup", "1", "--no-cpu-baseline", "--no-ceilings"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "kernels"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("tiny-zero2")
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert set(d["kernels"]) == {"reduce", "adam"}
    p = d["parity"]
    assert p["reduce_bit_exact"] is True and p["adam_bit_exact"] is True
    assert p["adam_steps"] == 3
    tr = d["trajectory"]
    assert (tr["live_steps"], tr["workload_steps"], tr["scratch_steps"]) == (3, 3, 3)
    assert d["dtype"] == "fp16-io/fp32-state"
    st = d["device_settle"]                  # the wait for a quiet device ran first
    assert st["reads"] >= 2 and 1.0 <= st["seconds"] < 20.0 and st["best_gbs"] > 0
