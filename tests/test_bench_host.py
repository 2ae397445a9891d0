"""bench.py's host logic on the CPU (no GPU needed): it refuses more than one GPU,
every workload choice maps to a workload, the counter summaries it reads for
roofline.traffic are looked up by kernel and workload and ignored once the kernel
source has changed, and every committed summary carries the fields it reads and a
command that runs committed files only."""
import hashlib
import importlib.util
import os
import re
import subprocess
import sys

import pytest

from conftest import ROOT


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120, cwd=ROOT,
                       env=dict(os.environ, **env))
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""


def test_every_workload_choice_maps_to_a_workload():
    b = _bench()
    names = {"zero2-7.5B-nd64": "zero2-7.5B-nd64-r0", "zero2-7.5B-nd64-g16": "zero2-7.5B-nd64-g16-r0",
             "zero3-7.5B-nd64": "zero3-7.5B-nd64-r0", "zero2-13B-nd32": "zero2-13B-nd32-r0",
             "zero2-100B-nd400": "zero2-100B-nd400-r137", "plain-dp-1.4B": "plain-dp-psi1400000000"}
    for arg, name in names.items():
        assert b.workload(arg, None).name == name
    assert b.workload("zero2-7.5B-nd64", 3).rank == 3
    assert b.workload("tiny-zero2", None).psi == 1 << 20
    assert b.workload("tiny-zero2", 3).rank == 3
    with pytest.raises(SystemExit):
        b.workload("plain-dp-1.4B", 1)


def _summary(dirpath, kernel, workload, sha, nbytes):
    path = os.path.join(dirpath, f"{kernel}__{workload}.md")
    with open(path, "w") as f:
        f.write(f"# {kernel} -- {workload}\n\n- measured HBM bytes per launch: {nbytes}\n"
                f"- kernel source sha256: `{sha}`\n")


def test_traffic_lookup_rules(tmp_path):
    b = _bench()
    sha = b.kernel_source_sha256("reduce_kernel")
    d = str(tmp_path)
    assert b.measured_traffic("reduce_kernel", "w1", d) is None           # no summary
    _summary(d, "reduce_kernel", "w1", sha, 123456)
    assert b.measured_traffic("reduce_kernel", "w1", d) == 123456
    _summary(d, "reduce_kernel", "w2", "0" * 64, 123456)                 # source changed since
    assert b.measured_traffic("reduce_kernel", "w2", d) is None
    _summary(d, "adam_vec_kernel", "w1", sha, 99)                        # another kernel's source
    assert b.measured_traffic("adam_vec_kernel", "w1", d) is None
    # the digest covers the kernel's source and the internal headers it compiles
    csrc = os.path.join(ROOT, "zero_sharded_mixed_bucketed_amd", "csrc")
    h = hashlib.sha256()
    for f in ["reduce_shard.hip"] + sorted(f for f in os.listdir(csrc) if f.endswith(".h")):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    assert sha == h.hexdigest()
    assert {"kernels.h", "reduce_plan.h", "gather_plan.h"} <= set(os.listdir(csrc))


def test_committed_summaries_match_the_current_sources():
    """Every committed rocprofv3 summary was taken from the kernel sources and
    headers as they stand, so the counter bytes the bench reports from it
    describe the code that runs."""
    b = _bench()
    pdir = os.path.join(ROOT, "profiles")
    for f in sorted(os.listdir(pdir)):
        if not f.endswith(".md"):
            continue
        kernel = f[:-3].split("__")[0]
        m = re.search(r"^- kernel source sha256: `([0-9a-f]{64})`$",
                      open(os.path.join(pdir, f)).read(), re.M)
        assert m and m.group(1) == b.kernel_source_sha256(kernel), f


def test_committed_summaries_are_well_formed():
    b = _bench()
    pdir = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(pdir) if f.endswith(".md")]
    assert files
    r = subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True)
    if r.returncode == 0:
        tracked = set(r.stdout.split())
    else:                                  # a copy of the tree without its history
        tracked = {p for p in ("bench.py",) if os.path.exists(os.path.join(ROOT, p))}
    choices = ("zero2-7.5B-nd64", "zero2-7.5B-nd64-g16", "zero3-7.5B-nd64", "zero2-13B-nd32",
               "zero2-100B-nd400", "plain-dp-1.4B", "tiny-zero2")
    names = {b.workload(c, None).name for c in choices}
    for f in files:
        kernel, workload = f[:-3].split("__")
        assert kernel in b.KERNEL_SOURCES, f
        assert workload in names, (f, "no bench workload has this name")
        text = open(os.path.join(pdir, f)).read()
        assert re.search(r"^- measured HBM bytes per launch: \d+$", text, re.M), f
        assert re.search(r"^- kernel source sha256: `[0-9a-f]{64}`$", text, re.M), f
        cmds = re.findall(r"rocprofv3 .* -- python3 (\S+)", text)
        assert cmds and all(c in tracked for c in cmds), (f, cmds)


def test_library_sources_digest_tracks_the_sources(tmp_path):
    b = _bench()
    d1 = b.library_sources_sha256()
    assert d1 == b.library_sources_sha256() and len(d1) == 64
    h = hashlib.sha256()
    for sub in ("include", os.path.join("zero_sharded_mixed_bucketed_amd", "csrc")):
        d = os.path.join(ROOT, sub)
        for f in sorted(os.listdir(d)):
            if f.endswith((".h", ".hip")):
                h.update(f.encode())
                h.update(open(os.path.join(d, f), "rb").read())
    assert d1 == h.hexdigest()


def test_host_cpu_model_is_named():
    """The CPU baseline's host is named in the JSON's env: the first 'model name' of
    /proc/cpuinfo, or None where the file has none."""
    model = _bench().host_cpu_model()
    with open("/proc/cpuinfo") as f:
        names = [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")]
    assert model == (names[0] if names else None)


def test_timed_steps_run_with_the_garbage_collector_off():
    """A full collection of Python's cyclic garbage collector (tens of ms on the host)
    between two timed steps leaves the GPU idle once the queued launches drain, so
    the collector is disabled from the warm-up to the end of the timed steps."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    main = src[src.index("def main():"):src.index("\ndef ", src.index("def main():") + 1)]
    off, warm = main.index("gc.disable()"), main.index("for _ in range(args.warmup):")
    timed, on = main.index("for k in range(args.steps):"), main.index("gc.enable()")
    assert off < warm < timed < on


def test_memory_busy_percent_reads_the_busiest_card(tmp_path, monkeypatch):
    """The quiet-device wait reads the driver's memory-busy counter of every card
    that exposes one and takes the highest; no such file gives None."""
    import glob as glob_mod
    import bench as b
    for card, val in (("card0", "3\n"), ("card1", "0\n"), ("card2", "junk\n")):
        d = tmp_path / card / "device"
        d.mkdir(parents=True)
        (d / "mem_busy_percent").write_text(val)
    real = glob_mod.glob
    monkeypatch.setattr(glob_mod, "glob", lambda pat: real(
        pat.replace("/sys/class/drm", str(tmp_path))))
    assert b.memory_busy_percent() == 3
    (tmp_path / "card0" / "device" / "mem_busy_percent").write_text("0")
    assert b.memory_busy_percent() == 0
    monkeypatch.setattr(glob_mod, "glob", lambda pat: [])
    assert b.memory_busy_percent() is None


def test_read_text(tmp_path):
    import bench as b
    f = tmp_path / "v"
    f.write_text("7.2.0\n")
    assert b.read_text(str(f)) == "7.2.0"
    assert b.read_text(str(tmp_path / "missing")) is None
