"""The path under HIP graph capture: one step (every bucket's reduce, then the
Adam step with its fp16 slot write) is captured once and replayed; each replay,
with eager work and synchronisations in between, must equal the same step run
eagerly, bit for bit.  The entry points allocate nothing, never synchronise and
use no memsets, so a caller can capture them (the scalars of the Adam step are
fixed at capture, so every replay is a step with the same t)."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_bucketed_amd as Z
from gpu_util import assert_bits, f32, need_gpu, rows_device, state_device, u16
from synth import gen, workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


def _setup(psi, nd, rank, bucket, seed):
    geom = Z.shard_geometry(psi, nd, rank)
    lo, n = geom.offset, geom.len
    buckets = []
    for off, blen in wl.buckets_touching(wl.uniform_buckets(psi, bucket), lo, lo + n):
        a, b = Z.bucket_intersect(geom, off, blen)
        buckets.append((a, b - a, rows_device(seed, nd, a, b - a, wl.Dist(1e-3))))
    state = [state_device(seed, lo, n, wl.Dist(0.02), gen.KIND_MASTER),
             state_device(seed, lo, n, wl.Dist(1e-4), gen.KIND_M),
             state_device(seed, lo, n, wl.Dist(1e-6, True), gen.KIND_V)]
    return geom, buckets, state


@pytest.mark.parametrize("g16", [False, True])
def test_captured_step_replays_equal_eager_steps(g16):
    psi, nd, rank, bucket, seed, replays = 1_000_003, 8, 3, 100_003, 31, 4
    geom, buckets, eager = _setup(psi, nd, rank, bucket, seed)
    _, _, graphed = _setup(psi, nd, rank, bucket, seed)
    dt = torch.int16 if g16 else torch.float32
    g_e = torch.zeros(geom.len, dtype=dt, device="cuda")
    g_g = torch.zeros(geom.len, dtype=dt, device="cuda")
    p_e = torch.zeros(psi, dtype=torch.int16, device="cuda")
    p_g = torch.zeros(psi, dtype=torch.int16, device="cuda")

    def step(state, grad, flat16, stream=None):
        for a, n, rows in buckets:
            if g16:
                Z.reduce_shard(geom, a, n, rows, None, grad, stream=stream)
            else:
                Z.reduce_shard(geom, a, n, rows, grad, stream=stream)
        Z.adam_step_shard(geom, *state, grad, flat16, 0, 1e-4, 0.9, 0.999, 1e-8, 1,
                          stream=stream)

    # warm the library (device attributes) and the allocator before capture
    scratch = [x.clone() for x in graphed]
    step(scratch, g_g.clone(), p_g.clone())
    torch.cuda.synchronize()
    del scratch

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(graphed, g_g, p_g, stream=side)
    torch.cuda.synchronize()
    # capturing enqueues nothing: the state is still the initial one
    assert_bits(f32(graphed[0]), f32(eager[0]), "state untouched by capture")

    noise = torch.randn(1 << 20, device="cuda")
    for r in range(replays):
        step(eager, g_e, p_e)
        graph.replay()
        noise = noise * 1.0001 + 1.0          # eager work between replays
        torch.cuda.synchronize()
        for a, b, name in zip(graphed, eager, ("master", "m", "v")):
            assert_bits(f32(a), f32(b), f"replay {r} {name}")
        if g16:
            assert_bits(u16(g_g), u16(g_e), f"replay {r} fp16 gradient shard")
        else:
            assert_bits(f32(g_g), f32(g_e), f"replay {r} gradient shard")
        assert_bits(u16(p_g), u16(p_e), f"replay {r} fp16 vector")
    assert np.isfinite(f32(noise)).all()


def test_captured_stage3_step_replays_equal_eager_steps():
    """Stage 3: every layer's parameters gathered in forward order, then again in
    reverse with the owned part of each layer's gradient reduced into the fp16
    shard, then Adam into the rank's own fp16 parameter shard (which the next
    step's gathers read), captured once and replayed."""
    psi, nd, rank, seed, replays = 600_011, 4, 1, 47, 3
    layers = [(0, 90_001), (90_001, 150_000), (240_001, 120_007), (360_008, 240_003)]
    geom = Z.shard_geometry(psi, nd, rank)
    lo, n = geom.offset, geom.len
    s_all = -(-psi // nd)
    rows = {}
    for off, ln in layers:
        a, b = Z.bucket_intersect(geom, off, ln)
        if a < b:
            rows[off] = (a, b - a, rows_device(seed, nd, a, b - a, wl.Dist(1e-3)))

    def state():
        shards = torch.empty((nd, s_all), dtype=torch.int16, device="cuda")
        shards.copy_(torch.from_numpy(
            np.random.default_rng(seed).integers(0, 0x3C00, size=(nd, s_all), dtype=np.int16)))
        return {"shards": shards,
                "master": state_device(seed, lo, n, wl.Dist(0.02), gen.KIND_MASTER),
                "m": state_device(seed, lo, n, wl.Dist(1e-4), gen.KIND_M),
                "v": state_device(seed, lo, n, wl.Dist(1e-6, True), gen.KIND_V),
                "grad": torch.zeros(n, dtype=torch.int16, device="cuda"),
                "layer": torch.zeros(max(ln for _, ln in layers), dtype=torch.int16,
                                     device="cuda")}

    def step(st, stream=None):
        for off, ln in layers:                                   # forward
            Z.gather_params(psi, nd, off, ln, st["shards"], st["layer"][:ln], stream=stream)
        for off, ln in reversed(layers):                         # backward
            Z.gather_params(psi, nd, off, ln, st["shards"], st["layer"][:ln], stream=stream)
            if off in rows:
                a, k, r = rows[off]
                Z.reduce_shard(geom, a, k, r, None, st["grad"], stream=stream)
        Z.adam_step_shard(geom, st["master"], st["m"], st["v"], st["grad"],
                          st["shards"][rank, :n], lo, 1e-4, 0.9, 0.999, 1e-8, 1, stream=stream)

    eager, graphed = state(), state()
    warm = state()
    step(warm)
    torch.cuda.synchronize()
    del warm
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(graphed, stream=side)
    torch.cuda.synchronize()
    for r in range(replays):
        step(eager)
        graph.replay()
        torch.cuda.synchronize()
        for key in ("master", "m", "v"):
            assert_bits(f32(graphed[key]), f32(eager[key]), f"replay {r} {key}")
        for key in ("grad", "shards", "layer"):
            assert_bits(u16(graphed[key]), u16(eager[key]), f"replay {r} {key}")


def test_captured_gather_across_many_shards():
    """A gather that crosses 37 shards takes three launches (at most 16 pieces
    each); captured once and replayed, it equals the oracle every time."""
    from oracle import stage3 as ost3
    psi, nd, lo, n, replays = 40_000, 37, 5, 39_990, 3
    s_all = -(-psi // nd)
    host = np.random.default_rng(5).integers(0, 1 << 16, size=(nd, s_all + 3), dtype=np.uint16)
    shards = torch.from_numpy(host.view(np.int16)).cuda()
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    Z.gather_params(psi, nd, lo, n, shards, out)            # warm-up, eager
    torch.cuda.synchronize()
    want = ost3.gather_params(host, psi, nd, lo, n)
    assert_bits(u16(out), want, "eager gather")
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        Z.gather_params(psi, nd, lo, n, shards, out, stream=side)
    torch.cuda.synchronize()
    for r in range(replays):
        out.fill_(0x7E01)
        graph.replay()
        torch.cuda.synchronize()
        assert_bits(u16(out), want, f"replay {r}")
