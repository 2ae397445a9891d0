#!/usr/bin/env python3
"""Throughput of the per-rank ZeRO-2 hot path on one MI355X.

One step = the whole path for one data-parallel rank: the owner's reduce of
every gradient bucket that meets its shard (buckets in arrival order, i.e.
reverse layer order), then one fused Adam step on the shard with the fp16 slot
write into the flat parameter vector.  Default workload: rank 0 of a 7.5B model
at Nd = 64 (shard of 117,187,500 elements; 25M-element buckets, five of which
meet the shard; fp16 gradients N(0, 1e-3); fp32 master N(0, 0.02), m N(0, 1e-4),
v |N(0, 1e-6)|; lr 1e-4, betas 0.9/0.999, eps 1e-8).  The Nd ranks' local
gradients of those buckets are synthetic and resident in HBM before timing.

Prints one JSON line: params/s of the whole step, HBM GB/s, per-kernel timings
from HIP events on the launch stream, the roofline of the dominant kernel, a
sampled self-check against the CPU oracle, and the oracle's own throughput on
the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_HBM_GBS = 8000.0
METRIC = "sharded Adam+reduce params/sec and achieved HBM GB/s (% of peak), 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="zero2-7.5B-nd64",
                    choices=["zero2-7.5B-nd64", "zero2-7.5B-nd64-g16", "zero2-13B-nd32",
                             "plain-dp-1.4B", "tiny-zero2"])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chunk", type=int, default=1 << 22,
                    help="shard elements per chunk of the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle work to time on the host (seconds, approximate)")
    ap.add_argument("--check-samples", type=int, default=4096)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (untimed) so that a counter "
                         "profile of this run holds a kernel of known traffic")
    return ap.parse_args()


def workload(name, rank):
    from synth import workloads as wl
    if name == "zero2-7.5B-nd64":
        return wl.zero2_7p5b(0 if rank is None else rank)
    if name == "zero2-7.5B-nd64-g16":
        return wl.zero2_7p5b_g16(0 if rank is None else rank)
    if name == "zero2-13B-nd32":
        return wl.zero2_13b(0 if rank is None else rank)
    if name == "plain-dp-1.4B":
        return wl.plain_dp_1p4b()
    return wl.tiny()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the path: the data-parallel ranks are "
              "simulated as Nd input rows on a single device, and no collective runs. "
              "Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import zero_sharded_mixed_bucketed_amd as Z
    from synth import device as sdev
    from synth import gen
    from synth import workloads as wl

    w = workload(args.workload, args.rank)
    geom = Z.shard_geometry(w.psi, w.nd, w.rank)
    S, lo = geom.len, geom.offset
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    print(f"[bench] workload {w.name}: psi={w.psi} nd={w.nd} rank={w.rank} shard=[{lo}, "
          f"+{S})", file=sys.stderr, flush=True)

    # ---- inputs resident in HBM (untimed) ----------------------------------------------
    with torch.cuda.stream(stream):
        master = torch.empty(S, dtype=torch.float32, device=dev)
        m = torch.empty_like(master)
        v = torch.empty_like(master)
        sdev.fill_state(master, w.seed, gen.KIND_MASTER, lo, w.master.sigma)
        sdev.fill_state(m, w.seed, gen.KIND_M, lo, w.m.sigma, w.m.absolute)
        sdev.fill_state(v, w.seed, gen.KIND_V, lo, w.v.sigma, w.v.absolute)
        param16 = torch.zeros(w.psi, dtype=torch.int16, device=dev)   # the flat fp16 vector
        buckets = []          # (flat offset, length, rows) for the buckets meeting the shard
        if w.fp16_grad:
            grad = torch.empty(S, dtype=torch.int16, device=dev)
            sdev.fill_grad_rows(grad.view(1, S), w.seed, lo, w.grad.sigma, w.grad.heavy_tail,
                                kind=gen.KIND_GRAD_FULL)
        else:
            g16 = w.grad_shard == "fp16"
            grad = torch.zeros(S, dtype=torch.int16 if g16 else torch.float32, device=dev)
            for off, n in wl.buckets_touching(w.buckets, lo, lo + S):
                a, b = Z.bucket_intersect(geom, off, n)
                stride = (b - a + 63) // 64 * 64     # rows start on 128-byte cache lines
                buf = torch.empty(w.nd * stride, dtype=torch.int16, device=dev)
                rows = buf.as_strided((w.nd, b - a), (stride, 1))
                sdev.fill_grad_rows(rows, w.seed, a, w.grad.sigma, w.grad.heavy_tail)
                buckets.append((a, b - a, rows))
    torch.cuda.synchronize()
    init_idx = None
    if args.check_samples:
        rng = np.random.default_rng(1)
        init_idx = np.unique(np.concatenate([
            np.arange(min(64, S)), np.arange(max(0, S - 64), S),
            rng.integers(0, S, size=args.check_samples)]))
    print(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 1e9:.2f} GB",
          file=sys.stderr, flush=True)

    if args.copy_calibration:
        # 2^28 fp32 elements: 1 GiB read and 1 GiB written by one plain copy kernel
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- one step of the path ------------------------------------------------------------
    t_counter = [0]

    def step(events=None):
        t_counter[0] += 1
        for i, (a, n, rows) in enumerate(buckets):
            if events is not None:
                events["reduce"][i][0].record(stream)
            if grad.dtype == torch.float32:
                Z.reduce_shard(geom, a, n, rows, grad, stream=stream)
            else:
                Z.reduce_shard(geom, a, n, rows, None, grad, stream=stream)
            if events is not None:
                events["reduce"][i][1].record(stream)
        if events is not None:
            events["adam"][0].record(stream)
        Z.adam_step_shard(geom, master, m, v, grad, param16, 0, w.lr, w.beta1, w.beta2, w.eps,
                          t_counter[0], stream=stream)
        if events is not None:
            events["adam"][1].record(stream)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per_step = [{"reduce": [(ev(), ev()) for _ in buckets], "adam": (ev(), ev())}
                for _ in range(args.steps)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(per_step[k])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    red_ms = [sum(a.elapsed_time(b) for a, b in e["reduce"]) for e in per_step]
    adam_ms = [e["adam"][0].elapsed_time(e["adam"][1]) for e in per_step]
    n_red_launch = len(buckets) * args.steps

    # algorithmic bytes: reduce reads 2 Nd and writes 4 bytes per owned element;
    # Adam reads g, master, m, v and writes master, m, v and the fp16 slot.
    g_bytes = 4 if grad.dtype == torch.float32 else 2     # gradient shard element
    red_bytes = S * (2 * w.nd + g_bytes) if buckets else 0
    adam_bytes = S * (26 + g_bytes)
    ms_step = total_ms / args.steps
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    red_avg = sum(red_ms) / args.steps
    adam_avg = sum(adam_ms) / args.steps
    kernels = {
        "adam": {"kernel": "adam_vec_kernel", "launches_per_step": 1,
                 "avg_ms": adam_avg, "min_ms": min(adam_ms),
                 "bytes_per_launch": adam_bytes, "bytes_per_element": adam_bytes / S,
                 "gbs": gbs(adam_bytes, adam_avg),
                 "frac_of_peak": gbs(adam_bytes, adam_avg) / PEAK_HBM_GBS,
                 "params_per_s": S / (adam_avg * 1e-3)},
    }
    if buckets:
        kernels["reduce"] = {
            "kernel": "reduce_kernel", "launches_per_step": len(buckets),
            "avg_ms_per_launch": sum(red_ms) / n_red_launch, "avg_ms_per_step": red_avg,
            "bytes_per_step": red_bytes, "bytes_per_element": 2 * w.nd + g_bytes,
            "gbs": gbs(red_bytes, red_avg), "frac_of_peak": gbs(red_bytes, red_avg) / PEAK_HBM_GBS,
            "params_per_s": S / (red_avg * 1e-3)}
    dom = max(kernels, key=lambda k: kernels[k].get("avg_ms_per_step", kernels[k].get("avg_ms")))
    dk = kernels[dom]
    dom_launch_ms = dk.get("avg_ms_per_launch", dk.get("avg_ms"))
    dom_launch_bytes = (red_bytes / len(buckets)) if dom == "reduce" else adam_bytes
    roofline = {"bound": "hbm", "kernel": dk["kernel"],
                "achieved": dom_launch_bytes / (dom_launch_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dom_launch_bytes / (dom_launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "traffic": measured_traffic(dk["kernel"], w.name),
                "algorithmic_bytes_per_launch": dom_launch_bytes}

    # ---- sampled self-check against the oracle (untimed) --------------------------------
    parity = None
    if init_idx is not None:
        parity = self_check(w, geom, buckets, grad, master, m, v, param16, init_idx,
                            t_counter[0])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, geom, args.cpu_chunk, args.cpu_seconds)

    step_bytes = red_bytes + adam_bytes
    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "hbm_gbs": gbs(step_bytes, ms_step),
        "hbm_frac_of_peak": gbs(step_bytes, ms_step) / PEAK_HBM_GBS,
        "bytes_per_step": step_bytes,
        "config": {"workload": w.name, "psi": w.psi, "nd": w.nd, "rank": w.rank,
                   "shard_elements": S, "buckets_in_shard": len(buckets),
                   "bucket_elements": wl.BUCKET, "grad": "fp16 rows" if buckets else "fp16",
                   "grad_shard": ("fp32" if g_bytes == 4 else "fp16") if buckets else None,
                   "state": "fp32 master/m/v", "slot": "fp16"},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


KERNEL_SOURCES = {"reduce_kernel": "reduce_shard.hip", "adam_vec_kernel": "adam_step_shard.hip"}


def kernel_source_sha256(kernel):
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "zero_sharded_mixed_bucketed_amd", "csrc", KERNEL_SOURCES[kernel])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(kernel, workload_name):
    """HBM bytes per launch from the committed counter summary of this kernel and
    workload, or None when there is none or the kernel source changed since."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"{kernel}__{workload_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    try:
        if fields["kernel source sha256"] != kernel_source_sha256(kernel):
            return None
        return int(fields["measured HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def self_check(w, geom, buckets, grad, master, m, v, param16, idx, steps_done):
    """Sampled comparison with the oracle: the reduced gradient bit for bit, and the
    state after all the bench's Adam steps, stepped by the oracle from the same
    initial values."""
    import torch
    from oracle import adam as oadam
    from oracle import reduce as ored
    from synth import gen
    flat = idx.astype(np.uint64) + np.uint64(geom.offset)
    it = torch.from_numpy(idx.astype(np.int64)).to(grad.device)
    if buckets:
        rows = np.stack([gen.grad_f16(w.seed, k, flat, w.grad.sigma, w.grad.heavy_tail)
                         for k in range(w.nd)])
        g_ref = ored.reduce_values(rows, w.nd)
        if grad.dtype == torch.float32:
            g_dev = grad.index_select(0, it).cpu().numpy()
            reduce_ok = bool(np.array_equal(g_ref.view(np.uint32), g_dev.view(np.uint32)))
        else:
            g_ref = g_ref.astype(np.float16).view(np.uint16)      # the fp16 gradient shard
            g_dev = grad.index_select(0, it).cpu().numpy().view(np.uint16)
            reduce_ok = bool(np.array_equal(g_ref, g_dev))
    else:
        g_ref = gen.grad_f16(w.seed, 0, flat, w.grad.sigma, w.grad.heavy_tail,
                             kind=gen.KIND_GRAD_FULL)
        reduce_ok = None
    th = gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma)
    mm = gen.state_f32(w.seed, gen.KIND_M, flat, w.m.sigma, w.m.absolute)
    vv = gen.state_f32(w.seed, gen.KIND_V, flat, w.v.sigma, w.v.absolute)
    for t in range(1, steps_done + 1):
        th, mm, vv, p16 = oadam.step_values(th, mm, vv, g_ref,
                                            oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t))
    got = [x.index_select(0, it).cpu().numpy() for x in (master, m, v)]
    pi = torch.from_numpy((idx + geom.offset).astype(np.int64)).to(grad.device)
    got_p = param16.index_select(0, pi).cpu().numpy().view(np.uint16)
    adam_ok = all(np.array_equal(a.view(np.uint32), b.view(np.uint32))
                  for a, b in zip(got, (th, mm, vv))) and np.array_equal(got_p, p16)
    rel = max(float(np.max(np.abs(a.astype(np.float64) - b) /
                           np.maximum(np.abs(b.astype(np.float64)), 1e-30)))
              for a, b in zip(got, (th, mm, vv)))
    return {"samples": int(idx.size), "adam_steps": steps_done,
            "reduce_bit_exact": reduce_ok, "adam_bit_exact": bool(adam_ok),
            "adam_max_rel_err": rel}


def _oracle_inputs(args):
    """Seeded inputs of one chunk of the shard for the oracle (host generator)."""
    from synth import gen
    w, lo, n = args
    flat = np.arange(lo, lo + n, dtype=np.uint64)
    th = gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma)
    mm = gen.state_f32(w.seed, gen.KIND_M, flat, w.m.sigma, w.m.absolute)
    vv = gen.state_f32(w.seed, gen.KIND_V, flat, w.v.sigma, w.v.absolute)
    if w.fp16_grad:
        g = gen.grad_f16(w.seed, 0, flat, w.grad.sigma, kind=gen.KIND_GRAD_FULL)
    else:
        g = np.stack([gen.grad_f16(w.seed, k, flat, w.grad.sigma, w.grad.heavy_tail)
                      for k in range(w.nd)])
    return th, mm, vv, g


def _oracle_time(w, inputs):
    from oracle import adam as oadam
    from oracle import reduce as ored
    th, mm, vv, g = inputs
    t0 = time.perf_counter()
    if not w.fp16_grad:
        g = ored.reduce_values(g, w.nd)
        if w.grad_shard == "fp16":
            g = g.astype(np.float16).view(np.uint16)
    t1 = time.perf_counter()
    oadam.step_values(th, mm, vv, g, oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, 1))
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def cpu_baseline(w, geom, chunk, target_s):
    """The oracle on the host, single-threaded, over consecutive chunks of the shard
    until about target_s seconds of oracle work (inputs are generated first, in a
    worker pool, and are not timed)."""
    import multiprocessing as mp
    first = _oracle_inputs((w, geom.offset, min(chunk, geom.len)))
    t_red, t_adam = _oracle_time(w, first)
    n_done = first[0].shape[0]
    del first
    per = max(t_red + t_adam, 1e-3)
    more = min(int(target_s / per), (geom.len - n_done) // chunk)
    if more > 0:
        jobs = [(w, geom.offset + n_done + i * chunk, chunk) for i in range(more)]
        workers = max(1, min(16, len(os.sched_getaffinity(0)) - 1, more))
        with mp.get_context("fork").Pool(workers) as pool:
            inputs = pool.map(_oracle_inputs, jobs)
        for inp in inputs:
            a, b = _oracle_time(w, inp)
            t_red, t_adam = t_red + a, t_adam + b
            n_done += inp[0].shape[0]
        del inputs
    total = t_red + t_adam
    what = "" if w.fp16_grad else f"reduce of {w.nd} fp16 rows + "
    return {"value": n_done / total, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_done} elements of the shard ({what}one Adam step), NumPy, "
                      f"one thread, {total:.1f} s of oracle work",
            "reduce_s": t_red, "adam_s": t_adam}


if __name__ == "__main__":
    main()
