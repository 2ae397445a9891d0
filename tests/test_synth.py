"""The seeded input generator and the workload geometry (CPU)."""
import json
import os

import numpy as np

from oracle import geometry as geo
from synth import gen, workloads as wl


def test_splitmix64_published_outputs(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "splitmix64_seed0.json")))
    got = gen.draws(0, np.arange(3))
    assert [int(x) for x in got] == [int(h, 16) for h in d["outputs"]]
    assert all(gen.mix64_int(((i + 1) * gen.GAMMA) & gen.MASK64) == int(h, 16)
               for i, h in enumerate(d["outputs"]))


def test_values_depend_only_on_flat_index():
    a = gen.grad_f16(1, 3, np.arange(1000, 3000, dtype=np.uint64), 1e-3)
    b = gen.grad_f16(1, 3, np.arange(2000, 2500, dtype=np.uint64), 1e-3)
    assert np.array_equal(a[1000:1500], b)
    assert not np.array_equal(gen.grad_f16(1, 4, np.arange(1000, 1500), 1e-3), b)


def test_tables():
    t = gen.table_f16(1e-3).view(np.float16).astype(np.float64)
    assert np.all(np.diff(t) >= 0)
    assert abs(t.mean()) < 1e-7 and abs(t.std() - 1e-3) < 2e-5
    t32 = gen.table_f32(0.02).astype(np.float64)
    assert np.all(np.diff(t32) > 0) and abs(t32.std() - 0.02) < 2e-4
    assert np.all(gen.table_f32(1e-6, absolute=True) >= 0)


def test_distributions():
    idx = np.arange(1 << 18, dtype=np.uint64)
    g = gen.grad_f16(2, 0, idx, 0.01).view(np.float16).astype(np.float64)
    assert abs(g.mean()) < 1e-4 and abs(g.std() - 0.01) < 2e-4
    h = gen.grad_f16(2, 0, idx, 1e-3, heavy_tail=True).view(np.float16).astype(np.float64)
    zero_frac = np.mean(h == 0)
    big = np.mean(np.abs(h) > 0.01)          # outliers are N(0, 0.1); normal values < 6e-3
    assert 0.009 < zero_frac < 0.011
    assert 0.008 < big < 0.011
    s = gen.state_f32(2, gen.KIND_MASTER, idx, 0.02)
    assert abs(s.std() - 0.02) < 3e-4
    assert np.all(gen.state_f32(2, gen.KIND_V, idx, 1e-6, absolute=True) >= 0)
    assert np.all(gen.state_f32(2, gen.KIND_M, idx, 0.0) == 0)


def test_uniform_bucket_geometry_7p5b():
    w = wl.zero2_7p5b(0)
    assert len(w.buckets) == 300
    assert w.buckets[0] == (7_500_000_000 - 25_000_000, 25_000_000)   # last layer first
    assert sum(n for _, n in w.buckets) == w.psi
    lo, hi = geo.shard_range(w.psi, w.nd, 0)
    touch = wl.buckets_touching(w.buckets, lo, hi)
    sizes = [geo.intersect(lo, hi, o, n) for o, n in touch]
    assert [b - a for a, b in sizes] == [17_187_500] + [25_000_000] * 4
    lo, hi = geo.shard_range(w.psi, w.nd, 1)
    touch = wl.buckets_touching(w.buckets, lo, hi)
    sizes = [b - a for a, b in (geo.intersect(lo, hi, o, n) for o, n in touch)]
    assert sizes == [9_375_000] + [25_000_000] * 4 + [7_812_500]
    assert (lo - touch[-1][0]) % 8 == 4      # rank 1 starts mid-way into a 16-byte group


def test_uniform_bucket_geometry_13b():
    w = wl.zero2_13b(0)
    assert len(w.buckets) == 520
    lo, hi = geo.shard_range(w.psi, w.nd, 0)
    sizes = [b - a for a, b in (geo.intersect(lo, hi, o, n)
                                for o, n in wl.buckets_touching(w.buckets, lo, hi))]
    assert sizes == [6_250_000] + [25_000_000] * 16


def test_transformer_bucket_geometry_100b():
    w = wl.zero2_100b(137)
    tensors = wl.transformer_tensors(w.psi, 8192)
    assert sum(n for _, n in tensors) == w.psi
    assert len(tensors) == 125 * 3 - 2          # 124 full layers + a truncated attention
    assert tensors[-1] == (124 * 805_322_752, 139_978_752)
    assert len(w.buckets) == 4222
    assert sum(n for _, n in w.buckets) == w.psi
    assert all(n <= wl.BUCKET for _, n in w.buckets)
    offs = [o for o, _ in w.buckets]
    assert offs == sorted(offs, reverse=True)   # reverse layer order
    lo, hi = geo.shard_range(w.psi, w.nd, w.rank)
    assert (lo, hi) == (34_250_000_000, 34_500_000_000)
    sizes = [b - a for a, b in (geo.intersect(lo, hi, o, n)
                                for o, n in wl.buckets_touching(w.buckets, lo, hi))]
    assert sizes == [21_138_048] + [25_000_000] * 9 + [3_861_952]
    # the shard lies inside layer 42's MLP tensor
    mlp = tensors[42 * 3 + 1]
    assert mlp[0] <= lo and hi <= mlp[0] + mlp[1]
