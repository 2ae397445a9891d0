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
Other workloads (--workload): the same step with an fp16 gradient shard, stage
3 with its per-layer parameter gathers, 13B at Nd = 32 with heavy-tailed
gradients, 100B at Nd = 400 (rank 137; 200 GB of gradient rows resident,
reduced in 2^22-column launches; the fp16 vector as a window around the slot),
plain data parallelism at 1.4B, and a tiny case.

Prints one JSON line: params/s of the whole step, HBM GB/s, per-kernel timings
from HIP events on the launch stream, the roofline of the dominant kernel, a
sampled self-check against the CPU oracle, and the oracle's own throughput on
the host as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rank R]
                    [--seed S] [--no-cpu-baseline] [--no-ceilings]
"""
from __future__ import annotations

import argparse
import dataclasses
import gc
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
                    choices=["zero2-7.5B-nd64", "zero2-7.5B-nd64-g16", "zero3-7.5B-nd64",
                             "zero2-13B-nd32", "zero2-100B-nd400", "plain-dp-1.4B",
                             "tiny-zero2"])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chunk", type=int, default=1 << 22,
                    help="shard elements per chunk of the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle work to time on the host (seconds, approximate)")
    ap.add_argument("--check-samples", type=int, default=4096)
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming ceilings reported for context")
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the wait for a quiet device before the warm-up steps")
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
    if name == "zero3-7.5B-nd64":
        return wl.zero3_7p5b(0 if rank is None else rank)
    if name == "zero2-13B-nd32":
        return wl.zero2_13b(0 if rank is None else rank)
    if name == "zero2-100B-nd400":
        return wl.zero2_100b(137 if rank is None else rank)
    if name == "plain-dp-1.4B":
        if rank not in (None, 0):
            raise SystemExit("plain data parallelism has one rank (Nd = 1): --rank 0")
        return wl.plain_dp_1p4b()
    return wl.tiny(rank=0 if rank is None else rank)


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
    if args.seed is not None:
        w = dataclasses.replace(w, seed=args.seed)
    stage3 = w.extra.get("stage") == 3
    geom = Z.shard_geometry(w.psi, w.nd, w.rank)
    S, lo = geom.len, geom.offset
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    print(f"[bench] workload {w.name}: psi={w.psi} nd={w.nd} rank={w.rank} shard=[{lo}, "
          f"+{S})", file=sys.stderr, flush=True)

    # ---- inputs resident in HBM (untimed) ----------------------------------------------
    # Generating them is not part of the metric; its time is reported on its own
    # (wall time with the allocations, and the device time of the generator
    # kernels on the stream between two events).
    shards = layer_buf = None
    torch.cuda.synchronize()
    setup_wall0 = time.perf_counter()
    setup_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    setup_ev[0].record(stream)
    with torch.cuda.stream(stream):
        # The reduce's rows are allocated first (the order does not change how
        # fast they read once the device is quiet; see the settle step below).
        buckets = []          # (flat offset, length, rows) per reduce launch
        n_buckets = 0         # buckets meeting the shard
        if not w.fp16_grad:
            chunk = w.extra.get("chunk")          # rows arrive in column chunks
            for off, n in wl.buckets_touching(w.buckets, lo, lo + S):
                a, b = Z.bucket_intersect(geom, off, n)
                n_buckets += 1
                for c0 in range(a, b, chunk or (b - a)):
                    c1 = min(b, c0 + (chunk or (b - a)))
                    stride = Z.row_stride(c1 - c0)
                    buf = torch.empty(w.nd * stride, dtype=torch.int16, device=dev)
                    rows = buf.as_strided((w.nd, c1 - c0), (stride, 1))
                    sdev.fill_grad_rows(rows, w.seed, c0, w.grad.sigma, w.grad.heavy_tail)
                    buckets.append((c0, c1 - c0, rows))
        if stage3:
            # every rank's fp16 parameter shard (the all-gather sources); row
            # `rank` is this rank's own shard, which its Adam step writes
            s_all = -(-w.psi // w.nd)
            shards = torch.empty((w.nd, s_all), dtype=torch.int16, device=dev)
            fill_param_shards(sdev, gen, w, shards)
            param16, param16_origin = shards[w.rank, :S], lo
            layer_buf = torch.empty(max(n for _, n in w.buckets), dtype=torch.int16, device=dev)
        live = RankArrays(torch, dev, S)
        live.fill_initial(sdev, gen, w, lo)
        if w.fp16_grad:
            grad = torch.empty(S, dtype=torch.int16, device=dev)
            sdev.fill_grad_rows(grad.view(1, S), w.seed, lo, w.grad.sigma, w.grad.heavy_tail,
                                kind=gen.KIND_GRAD_FULL)
        else:
            grad = torch.zeros(S, dtype=torch.int16 if w.grad_shard == "fp16" else torch.float32,
                               device=dev)
        if stage3:
            pass                                  # the slot is the own parameter shard
        elif "p16_window" in w.extra:
            # the rank's slot and a margin either side of it, at its place in the
            # flat fp16 vector (the whole vector does not fit beside the rows)
            win = w.extra["p16_window"]
            param16_origin = max(0, lo - win)
            param16 = torch.zeros(min(w.psi, lo + S + win) - param16_origin, dtype=torch.int16,
                                  device=dev)
        else:
            param16, param16_origin = torch.zeros(w.psi, dtype=torch.int16, device=dev), 0
        live.set_slot(param16, param16_origin)
        # Scratch state for the warm-up steps and for timed steps beyond the
        # workload's own count: Adam updates in place, so those steps run on
        # copies and the live state follows exactly the workload's trajectory
        # t = 1..K.  The scratch fp16 slot sits at the live slot's address
        # modulo 256 bytes, so both take the same store widths.
        scratch = RankArrays(torch, dev, S)
        scratch.copy_from(live)
        slot_ptr = param16.data_ptr() + 2 * (lo - param16_origin)
        sbuf = torch.empty(S + 128, dtype=torch.int16, device=dev)
        e = ((slot_ptr - sbuf.data_ptr()) % 256) // 2
        scratch.set_slot(sbuf[e:e + S], lo)
    setup_ev[1].record(stream)
    torch.cuda.synchronize()
    input_setup = {"wall_s": time.perf_counter() - setup_wall0,
                   "device_ms": setup_ev[0].elapsed_time(setup_ev[1]),
                   "bytes_resident": torch.cuda.memory_allocated(),
                   "what": "seeded synthetic inputs generated on the device (untimed, not in "
                           "value); gradient rows allocated first, then the model state"}
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

    # ---- one step of the path: a list of launches -----------------------------------------
    # Algorithmic bytes per launch: the reduce reads 2 Nd and writes the gradient
    # element (4 or 2 bytes) per owned column; Adam reads g, master, m, v and
    # writes master, m, v and the fp16 parameter (26 bytes + the gradient); a
    # parameter gather reads and writes 2 bytes per element.
    g_bytes = 4 if grad.dtype == torch.float32 else 2
    red_of = {a: rows for a, _, rows in buckets}

    def launches(t, st):
        """The launches of step t on the rank arrays `st` (live or scratch)."""
        ops = []

        def reduce_op(a, n, rows):
            if grad.dtype == torch.float32:
                return lambda: Z.reduce_shard(geom, a, n, rows, grad, stream=stream)
            return lambda: Z.reduce_shard(geom, a, n, rows, None, grad, stream=stream)

        if stage3:
            layers = list(reversed(w.buckets))                   # forward order
            for off, n in layers:                                # forward gathers
                ops.append(("gather", n * 4, lambda off=off, n=n: Z.gather_params(
                    w.psi, w.nd, off, n, shards, layer_buf[:n], stream=stream)))
            for off, n in w.buckets:                             # backward, reverse order
                ops.append(("gather", n * 4, lambda off=off, n=n: Z.gather_params(
                    w.psi, w.nd, off, n, shards, layer_buf[:n], stream=stream)))
                a, b = Z.bucket_intersect(geom, off, n)
                if a < b:
                    ops.append(("reduce", (b - a) * (2 * w.nd + g_bytes),
                                reduce_op(a, b - a, red_of[a])))
        else:
            for a, n, rows in buckets:
                ops.append(("reduce", n * (2 * w.nd + g_bytes), reduce_op(a, n, rows)))
        ops.append(("adam", S * (26 + g_bytes), lambda: Z.adam_step_shard(
            geom, st.master, st.m, st.v, grad, st.p16, st.p16_origin, w.lr, w.beta1, w.beta2,
            w.eps, t, stream=stream)))
        return ops

    def runs_of(ops):
        """Consecutive launches of one kernel kind: [(kind, launches), ...]."""
        runs = []
        for kind, _, _ in ops:
            if runs and runs[-1][0] == kind:
                runs[-1][1] += 1
            else:
                runs.append([kind, 1])
        return runs

    def step(t, st, events=None):
        """Step t on `st`; with events, one is recorded before each run of
        launches of one kind and one after the step's last launch."""
        ops = launches(t, st)
        prev, r = None, 0
        for kind, _, fn in ops:
            if events is not None and kind != prev:
                events[r].record(stream)
                r, prev = r + 1, kind
            fn()
        if events is not None:
            events[r].record(stream)
        return ops

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # Wait for a quiet device (the driver clears freed device memory in the
    # background, which slows concurrent kernels for seconds).
    settle = None if args.no_settle else settle_device(
        torch, stream, buckets[max(range(len(buckets)), key=lambda i: buckets[i][1])][2]
        if buckets else live.master)

    # Python's cyclic garbage collector stays off from the warm-up to the end of
    # the timed steps: a full collection takes tens of milliseconds on the host,
    # and one falling between two timed steps left the GPU idle for as long once
    # the launches already queued had drained.
    # The live state takes steps t = 1..K of the workload (K = its own step
    # count, or fewer when fewer steps are timed); warm-ups and timed steps past
    # K run on the scratch copy, which continues its own count.
    k_live = min(args.steps, w.steps)
    t_scratch = 0
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        t_scratch += 1
        step(t_scratch, scratch)
    torch.cuda.synchronize()
    # The timed steps: besides the path's own launches the stream holds only the
    # events at the boundaries of each run of one kernel kind (3 per step for
    # stage 2), so the per-kernel figures come from the timed region itself.
    runs = runs_of(launches(1, live))
    per_step = [[ev() for _ in range(len(runs) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ops = None
    for k in range(args.steps):
        if k < k_live:
            ops = step(k + 1, live, per_step[k])
        else:
            t_scratch += 1
            ops = step(t_scratch, scratch, per_step[k])
    enqueued = time.perf_counter() - wall0         # host time to issue the timed steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    total_ms = per_step[0][0].elapsed_time(per_step[-1][-1])
    ms_step = total_ms / args.steps

    # ---- per-kernel figures from the run events ----------------------------------------
    names = {"reduce": "reduce_kernel", "adam": "adam_vec_kernel", "gather": "copy_kernel"}
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    kernels = {}
    for kind in dict.fromkeys(k for k, _ in runs):
        rs = [r for r, (k, _) in enumerate(runs) if k == kind]
        n_launch = sum(runs[r][1] for r in rs)
        bytes_step = sum(b for k, b, _ in ops if k == kind)
        per = [sum(per_step[s][r].elapsed_time(per_step[s][r + 1]) for r in rs)
               for s in range(args.steps)]
        avg_step = sum(per) / args.steps
        kernels[kind] = {
            "kernel": names[kind], "launches_per_step": n_launch,
            "avg_ms_per_launch": avg_step / n_launch, "avg_ms_per_step": avg_step,
            "min_ms_per_step": min(per), "median_ms_per_step": float(np.median(per)),
            "bytes_per_step": bytes_step,
            "bytes_per_element": bytes_step / S,
            "gbs": gbs(bytes_step, avg_step), "frac_of_peak": gbs(bytes_step, avg_step) / PEAK_HBM_GBS,
            "params_per_s": S / (avg_step * 1e-3)}
        traffic = measured_traffic(names[kind], w.name)
        kernels[kind]["counter_bytes_per_launch"] = traffic
        kernels[kind]["counter_bytes_per_element"] = (
            traffic * n_launch / S if traffic is not None else None)
        kernels[kind]["waves_per_cu_measured"] = measured_waves_per_cu(names[kind], w.name)
        kernels[kind]["workgroups_per_cu_cap"] = {
            "reduce": lambda: Z.launch_occupancy(Z.KERNEL_REDUCE_W16)[0],
            "adam": lambda: Z.launch_occupancy(Z.KERNEL_ADAM_G32 if g_bytes == 4
                                               else Z.KERNEL_ADAM_G16)[0],
            "gather": lambda: None}[kind]()
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms_per_step"])
    dk = kernels[dom]
    dom_launch_bytes = dk["bytes_per_step"] / dk["launches_per_step"]
    achieved = gbs(dom_launch_bytes, dk["avg_ms_per_launch"])
    roofline = {"bound": "hbm", "kernel": dk["kernel"], "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(dk["kernel"], w.name),
                "algorithmic_bytes_per_launch": dom_launch_bytes}

    # ---- sampled self-check against the oracle (untimed) --------------------------------
    parity = None
    if init_idx is not None:
        parity = self_check(w, geom, buckets, grad, live.master, live.m, live.v, param16,
                            param16_origin, init_idx, k_live)
        if stage3:
            parity.update(gather_check(w, geom, shards, layer_buf, init_idx, k_live, stream))

    ceilings = None
    if not args.no_ceilings:
        widest = max(buckets, key=lambda b: b[1], default=None)
        ceilings = stream_ceilings(torch, dev, stream, widest[2] if widest else None)
        if "reduce" in kernels and "read_rows_gbs" in ceilings:
            ceilings["reduce_of_read_rows"] = kernels["reduce"]["gbs"] / ceilings["read_rows_gbs"]

    cpu = None
    if not args.no_cpu_baseline:
        # at most 2^28 fp16 gradient values per oracle chunk (512 MiB of host memory)
        cpu_chunk = max(1 << 10, min(args.cpu_chunk, (1 << 28) // w.nd))
        cpu = cpu_baseline(w, geom, cpu_chunk, args.cpu_seconds)

    step_bytes = sum(k["bytes_per_step"] for k in kernels.values())
    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "host_enqueue_ms_per_step": enqueued * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16-io/fp32-state", "data": "synthetic",
        "hbm_gbs": gbs(step_bytes, ms_step),
        "hbm_frac_of_peak": gbs(step_bytes, ms_step) / PEAK_HBM_GBS,
        "bytes_per_step": step_bytes,
        "config": {"workload": w.name, "psi": w.psi, "nd": w.nd, "rank": w.rank,
                   "seed": w.seed,
                   "stage": 3 if stage3 else (1 if w.nd == 1 else 2),
                   "shard_elements": S, "buckets_in_shard": n_buckets,
                   "reduce_launches": len(buckets),
                   "bucket_elements": ("layer" if stage3 else
                                       max((n for _, n in w.buckets), default=None)),
                   "chunk_elements": w.extra.get("chunk"),
                   "grad": "fp16 rows" if buckets else "fp16",
                   "grad_shard": ("fp32" if g_bytes == 4 else "fp16") if buckets else None,
                   "state": "fp32 master/m/v",
                   "slot": ("own fp16 shard" if stage3 else
                            "fp16 flat vector window" if "p16_window" in w.extra else
                            "fp16 flat vector")},
        "trajectory": {"live_steps": k_live, "workload_steps": w.steps,
                       "scratch_steps": args.warmup + args.steps - k_live,
                       "what": "the live state takes steps t = 1..live_steps; warm-ups and "
                               "timed steps past the workload's count run on a scratch copy "
                               "of master/m/v and of the fp16 slot"},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "ceilings": ceilings,
        "input_setup": input_setup,
        "device_settle": settle,
        "env": environment(torch, dev),
    }
    print(json.dumps(out), flush=True)


class RankArrays:
    """The rank's Adam state (fp32 master, m, v) and the fp16 slot its step writes."""

    def __init__(self, torch, dev, n):
        self.master = torch.empty(n, dtype=torch.float32, device=dev)
        self.m = torch.empty_like(self.master)
        self.v = torch.empty_like(self.master)
        self.p16, self.p16_origin = None, 0

    def fill_initial(self, sdev, gen, w, lo):
        sdev.fill_state(self.master, w.seed, gen.KIND_MASTER, lo, w.master.sigma)
        sdev.fill_state(self.m, w.seed, gen.KIND_M, lo, w.m.sigma, w.m.absolute)
        sdev.fill_state(self.v, w.seed, gen.KIND_V, lo, w.v.sigma, w.v.absolute)

    def copy_from(self, other):
        for a, b in ((self.master, other.master), (self.m, other.m), (self.v, other.v)):
            a.copy_(b)

    def set_slot(self, p16, origin):
        self.p16, self.p16_origin = p16, origin


def fill_param_shards(sdev, gen, w, shards):
    """Stage 3: every rank's fp16 parameter shard, row k = rank k's."""
    s_all = shards.shape[1]
    for k in range(w.nd):
        k_lo = min(k * s_all, w.psi)
        k_n = min((k + 1) * s_all, w.psi) - k_lo
        if k_n:
            sdev.fill_grad_rows(shards[k:k + 1, :k_n], w.seed, k_lo, w.extra["param_sigma"],
                                rank0=k, kind=gen.KIND_PARAM16)


def memory_busy_percent():
    """The memory controller's busy percentage the driver reports in sysfs, the
    highest over the cards that expose it, or None where none does."""
    import glob
    vals = []
    for path in glob.glob("/sys/class/drm/card*/device/mem_busy_percent"):
        try:
            with open(path) as f:
                vals.append(int(f.read().strip()))
        except (OSError, ValueError):
            pass
    return max(vals) if vals else None


def settle_device(torch, stream, data, quiet_s=1.0, max_s=30.0, period_s=0.1):
    """Wait, before the warm-ups, until nothing else moves data on the device.

    The driver clears freed device memory in the background; after a process
    frees tens of GB (the previous run's exit does), concurrent kernels stream
    1-5% slower for seconds.  First, with this process idle, the memory
    controller's busy percentage (sysfs mem_busy_percent) must read 0 for half
    a second.  Then untimed reads of `data` (the workload's own resident data,
    read as 64 or more rows) run back to back, timed in batches of about 20 GB,
    until the rate has not risen by more than 0.3% for `quiet_s` seconds; the
    device is then busy and clocked up when the warm-ups start.  Both waits
    stop at `max_s`."""
    from synth import probe
    t0 = time.perf_counter()
    idle_reads, busy_seen = 0, []
    while time.perf_counter() - t0 < max_s:
        b = memory_busy_percent()
        if b is None:                      # not exposed here: the read check alone
            break
        busy_seen.append(b)
        idle_reads = idle_reads + 1 if b == 0 else 0
        if idle_reads >= 5:
            break
        time.sleep(period_s)
    t_idle = time.perf_counter() - t0
    if data.dim() == 2 and data.dtype == torch.int16:
        view = data[:, :data.shape[1] // 8 * 8]
    else:
        flat = data.view(torch.int16)
        cols = flat.numel() // 64 // 8 * 8
        view = flat[:64 * cols].view(64, cols)
    with torch.cuda.stream(stream):
        sink = torch.zeros(1, dtype=torch.int32, device=data.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    nbytes = 2 * view.shape[0] * view.shape[1]
    reps = max(1, int(2e10 // nbytes))     # about 20 GB (3 ms) per timed batch
    t1 = time.perf_counter()
    rates, best, t_best = [], 0.0, t1
    while True:                            # back to back: the device stays busy
        with torch.cuda.stream(stream):
            ev[0].record(stream)
            for _ in range(reps):
                probe.read_rows(view, sink, 8, stream=stream)
            ev[1].record(stream)
        torch.cuda.synchronize()
        r = reps * nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
        rates.append(r)
        now = time.perf_counter()
        if r > best * 1.003:
            best, t_best = r, now
        if now - t_best >= quiet_s or now - t1 >= max_s:
            break
    return {"seconds": time.perf_counter() - t0, "memory_idle_wait_s": t_idle,
            "memory_busy_max": max((b for b in busy_seen if b is not None), default=None),
            "reads": len(rates), "first_gbs": rates[0], "best_gbs": best,
            "what": "before the warm-ups: wait until the driver reports the memory controller "
                    "idle, then read the workload's resident data back to back, untimed, until "
                    "the rate stops rising (the driver clears freed device memory in the "
                    "background)"}


def stream_ceilings(torch, dev, stream, rows=None, nbytes=4 << 30, reps=10):
    """Practical HBM rates on the same box, timed with HIP events on the launch
    stream after the measurement; context for the kernels' rates.

    - read_rows: the reduce's access pattern, without its arithmetic and stores,
      at the reduce's occupancy cap, over the very rows of the workload's widest
      reduce launch (their first columns, a multiple of 8, at most nbytes): the
      read rate of one allocation moves by several per cent with where it lands,
      so the reduce is compared with a read of the same memory;
    - write, copy: 16-byte stores / non-temporal loads and stores over nbytes,
      no occupancy cap;
    - runtime_copy, runtime_fill: torch's own device copy_ and fill_ over nbytes.
    """
    from synth import probe

    def timed(fn):
        with torch.cuda.stream(stream):
            fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    gbs = lambda moved, ms: moved / (ms * 1e-3) / 1e9
    out = {}
    if rows is not None:
        nd, cols = rows.shape
        cols = min(cols, nbytes // (2 * nd)) // 8 * 8
        view = rows[:, :cols]
        with torch.cuda.stream(stream):
            sink = torch.zeros(1, dtype=torch.int32, device=dev)
        ms = timed(lambda: probe.read_rows(view, sink, 8, stream=stream))
        out["read_rows_gbs"] = gbs(2 * nd * cols, ms)
        out["read_rows_shape"] = [nd, cols, rows.stride(0)]
        out["read_rows_source"] = "the rows of the widest reduce launch"
        del view, sink
    n = nbytes // 4
    with torch.cuda.stream(stream):
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for name, fn, moved in (("write", lambda c: probe.write(dst, c, stream=stream), nbytes),
                            ("copy", lambda c: probe.copy(src, dst, c, stream=stream),
                             2 * nbytes)):
        out[f"{name}_gbs"] = gbs(moved, timed(lambda: fn(0)))
    out["runtime_copy_gbs"] = gbs(2 * nbytes, timed(lambda: dst.copy_(src)))
    out["runtime_fill_gbs"] = gbs(nbytes, timed(lambda: dst.fill_(1.5)))
    del src, dst
    torch.cuda.empty_cache()
    return out


def environment(torch, dev):
    """What the numbers were measured on."""
    p = torch.cuda.get_device_properties(dev)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "hbm_bytes": p.total_memory,
            "hip": torch.version.hip, "torch": torch.__version__,
            "numpy": np.__version__, "host_cpus": len(os.sched_getaffinity(0)),
            "rocm": read_text("/opt/rocm/.info/version"),
            "amdgpu_driver": read_text("/sys/module/amdgpu/version"),
            "host_cpu_model": host_cpu_model(),
            "library_sources_sha256": library_sources_sha256()}


def read_text(path):
    """A one-line version file's contents, or None."""
    try:
        with open(path) as f:
            return f.read().strip() or None
    except OSError:
        return None


def host_cpu_model():
    """The host CPU's model name (the oracle baseline runs on it), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def library_sources_sha256():
    """One digest over the library's header and HIP sources: which build ran."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    paths = []
    for d in (os.path.join(here, "include"),
              os.path.join(here, "zero_sharded_mixed_bucketed_amd", "csrc")):
        paths += [os.path.join(d, f) for f in sorted(os.listdir(d)) if f.endswith((".h", ".hip"))]
    for path in paths:
        h.update(os.path.basename(path).encode())
        h.update(open(path, "rb").read())
    return h.hexdigest()


KERNEL_SOURCES = {"reduce_kernel": "reduce_shard.hip", "adam_vec_kernel": "adam_step_shard.hip",
                  "copy_kernel": "gather_params.hip"}


def kernel_source_sha256(kernel):
    """One digest over the kernel's HIP source and the library's internal headers
    that every kernel source compiles (csrc/*.h: launch constants and the index
    plans), each file's name then its bytes: a profile recorded under another
    digest was taken from other code."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "zero_sharded_mixed_bucketed_amd", "csrc")
    paths = [os.path.join(csrc, KERNEL_SOURCES[kernel])]
    paths += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith(".h")]
    h = hashlib.sha256()
    for path in paths:
        h.update(os.path.basename(path).encode())
        h.update(open(path, "rb").read())
    return h.hexdigest()


def profile_fields(kernel, workload_name, profiles_dir=None):
    """The committed rocprofv3 summary of this kernel and workload, as its "- key:
    value" fields, or {} when there is none or the kernel source changed since."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(profiles_dir or os.path.join(here, "profiles"),
                        f"{kernel}__{workload_name}.md")
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != kernel_source_sha256(kernel):
        return {}
    return fields


def measured_traffic(kernel, workload_name, profiles_dir=None):
    """HBM bytes per launch from the committed counter summary of this kernel and
    workload, or None when there is none or the kernel source changed since."""
    try:
        return int(profile_fields(kernel, workload_name, profiles_dir)
                   ["measured HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def measured_waves_per_cu(kernel, workload_name, profiles_dir=None):
    """Mean resident waves per CU from the committed occupancy pass, or None."""
    v = profile_fields(kernel, workload_name, profiles_dir).get("mean waves resident per CU")
    try:
        return float(v.split()[0]) if v else None
    except ValueError:
        return None


def _oracle_after(w, flat, steps_done, buckets, fp16_shard):
    """The oracle at flat indices of the shard: the reduced gradient (fp32, or its
    fp16 bits for an fp16 shard; the raw fp16 gradient without buckets) and the
    state after `steps_done` Adam steps from the seeded initial state."""
    from oracle import adam as oadam
    from oracle import reduce as ored
    from synth import gen
    if buckets:
        rows = np.stack([gen.grad_f16(w.seed, k, flat, w.grad.sigma, w.grad.heavy_tail)
                         for k in range(w.nd)])
        g_ref = ored.reduce_values(rows, w.nd)
        if fp16_shard:
            g_ref = g_ref.astype(np.float16).view(np.uint16)
    else:
        g_ref = gen.grad_f16(w.seed, 0, flat, w.grad.sigma, w.grad.heavy_tail,
                             kind=gen.KIND_GRAD_FULL)
    th = gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma)
    mm = gen.state_f32(w.seed, gen.KIND_M, flat, w.m.sigma, w.m.absolute)
    vv = gen.state_f32(w.seed, gen.KIND_V, flat, w.v.sigma, w.v.absolute)
    p16 = None
    for t in range(1, steps_done + 1):
        th, mm, vv, p16 = oadam.step_values(th, mm, vv, g_ref,
                                            oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t))
    return g_ref, th, mm, vv, p16


def self_check(w, geom, buckets, grad, master, m, v, param16, param16_origin, idx, steps_done):
    """Sampled comparison with the oracle: the reduced gradient bit for bit, and the
    state after all the bench's Adam steps, stepped by the oracle from the same
    initial values."""
    import torch
    flat = idx.astype(np.uint64) + np.uint64(geom.offset)
    it = torch.from_numpy(idx.astype(np.int64)).to(grad.device)
    fp16_shard = grad.dtype != torch.float32
    g_ref, th, mm, vv, p16 = _oracle_after(w, flat, steps_done, buckets, fp16_shard)
    reduce_ok = None
    if buckets:
        g_dev = grad.index_select(0, it).cpu().numpy()
        reduce_ok = bool(np.array_equal(g_ref.view(np.uint16 if fp16_shard else np.uint32),
                                        g_dev.view(np.uint16 if fp16_shard else np.uint32)))
    got = [x.index_select(0, it).cpu().numpy() for x in (master, m, v)]
    pi = torch.from_numpy((idx + geom.offset - param16_origin).astype(np.int64)).to(grad.device)
    got_p = param16.index_select(0, pi).cpu().numpy().view(np.uint16)
    adam_ok = all(np.array_equal(a.view(np.uint32), b.view(np.uint32))
                  for a, b in zip(got, (th, mm, vv))) and np.array_equal(got_p, p16)
    rel = max(float(np.max(np.abs(a.astype(np.float64) - b) /
                           np.maximum(np.abs(b.astype(np.float64)), 1e-30)))
              for a, b in zip(got, (th, mm, vv)))
    return {"samples": int(idx.size), "adam_steps": steps_done,
            "reduce_bit_exact": reduce_ok, "adam_bit_exact": bool(adam_ok),
            "adam_max_rel_err": rel}


def gather_check(w, geom, shards, layer_buf, idx, steps_done, stream):
    """Stage 3: gather (untimed) the layer holding the end of the rank's shard and
    compare sampled elements with the oracle: inside the shard, the fp16
    parameters after the bench's Adam steps; elsewhere, the other ranks' shards
    as generated."""
    import torch
    import zero_sharded_mixed_bucketed_amd as Z
    from synth import gen
    last = geom.offset + geom.len - 1
    off, n = next((o, k) for o, k in w.buckets if o <= last < o + k)
    with torch.cuda.stream(stream):
        Z.gather_params(w.psi, w.nd, off, n, shards, layer_buf[:n], stream=stream)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rel = np.unique(np.concatenate([np.arange(min(64, n)), np.arange(max(0, n - 64), n),
                                    np.clip(np.arange(last - off - 63, last - off + 65), 0, n - 1),
                                    rng.integers(0, n, size=idx.size)])).astype(np.int64)
    flat = (rel + off).astype(np.uint64)
    got = layer_buf.index_select(0, torch.from_numpy(rel).to(layer_buf.device)).cpu().numpy() \
        .view(np.uint16)
    # each gathered element is its owner's current fp16 parameter: inside this
    # rank's shard, the oracle's after the Adam steps; elsewhere, as generated
    s_all = -(-w.psi // w.nd)
    owner = (flat // np.uint64(s_all)).astype(np.int64)
    want = np.empty(flat.size, np.uint16)
    mine = owner == geom.rank
    if mine.any():
        want[mine] = _oracle_after(w, flat[mine], steps_done, True, True)[4]
    for k in np.unique(owner[~mine]):
        sel = owner == k
        want[sel] = gen.grad_f16(w.seed, int(k), flat[sel], w.extra["param_sigma"],
                                 kind=gen.KIND_PARAM16)
    return {"gather_samples": int(rel.size), "gather_bit_exact": bool(np.array_equal(got, want)),
            "gather_layer": [int(off), int(n)]}


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
    worker pool, and are not timed).  Worker pools start fresh interpreters
    ("spawn"): a forked child would inherit this process's GPU state."""
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
        with mp.get_context("spawn").Pool(workers) as pool:
            inputs = pool.map(_oracle_inputs, jobs)
        for inp in inputs:
            a, b = _oracle_time(w, inp)
            t_red, t_adam = t_red + a, t_adam + b
            n_done += inp[0].shape[0]
        del inputs
    total = t_red + t_adam
    what = "" if w.fp16_grad else f"reduce of {w.nd} fp16 rows + "
    out = {"value": n_done / total, "unit": "params/s", "cores": 1, "kind": "oracle",
           "sample": f"first {n_done} elements of the shard ({what}one Adam step), NumPy, "
                     f"one thread, {total:.1f} s of oracle work",
           "reduce_s": t_red, "adam_s": t_adam}
    out["all_cores"] = cpu_baseline_all_cores(w, geom, chunk)
    return out


def _oracle_chunk_timed(args):
    """In a worker: generate one chunk's inputs (untimed), then time the oracle on it."""
    w, lo, n = args
    t_red, t_adam = _oracle_time(w, _oracle_inputs((w, lo, n)))
    return os.getpid(), n, t_red + t_adam


def cpu_baseline_all_cores(w, geom, chunk, chunks_per_worker=2):
    """The same unchanged oracle over chunks in one process per host core (the work
    is element-wise, so chunks are independent): elements over the busiest worker's
    oracle time.  Each worker takes about `chunks_per_worker` chunks."""
    import multiprocessing as mp
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    n_chunks = min(workers * chunks_per_worker, -(-geom.len // chunk))
    jobs = [(w, geom.offset + i * chunk, min(chunk, geom.len - i * chunk)) for i in range(n_chunks)]
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_oracle_chunk_timed, jobs, chunksize=1)
    busy = {}
    for pid, _, t in res:
        busy[pid] = busy.get(pid, 0.0) + t
    n = sum(r[1] for r in res)
    return {"value": n / max(busy.values()), "unit": "params/s", "cores": len(busy),
            "kind": "oracle",
            "sample": f"{n} elements of the shard in {len(jobs)} chunks over {len(busy)} "
                      f"processes; elements / the busiest process's oracle time"}


if __name__ == "__main__":
    main()
