"""Pins of oracle.reduce.

* Closed form: fp16 values are integer multiples of 2^-24, so while every
  partial sum stays below 1 in magnitude the fp32 running sum is exact, and the
  result must equal RN32(exact integer sum * RN32(1/Nd)) whatever the order.
* Hand-worked IEEE cases where the order, the start value, the scale or the
  fp16 rounding changes the bits (tests/golden/reduce_order_cases.json).
* Brute force over all ranks of tiny models: the union of the shards is the
  full mean gradient; nothing outside a bucket/shard intersection is written.
"""
import json
import os

import numpy as np
import pytest

from oracle import geometry as geo
from oracle import reduce as red
from synth import gen


def _exact_reference(rows, nd):
    """(expected fp32, mask of elements whose partial sums all stay below 1)."""
    units = (rows.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    prefix = np.cumsum(units, axis=0)
    ok = np.all(np.abs(prefix) < (1 << 24), axis=0)
    total = prefix[-1].astype(np.float64) * 2.0 ** -24           # exact
    inv = float(np.float32(1.0) / np.float32(nd))
    # the product of two 24-bit significands is exact in fp64; one rounding to fp32
    return (total * inv).astype(np.float32), ok


@pytest.mark.parametrize("nd,sigma", [(4, 0.01), (64, 1e-3), (32, 1e-3), (3, 0.01),
                                      (400, 1e-3), (7, 0.05)])
def test_closed_form(nd, sigma):
    n = 4096 if nd >= 64 else 20000
    rows = gen.grad_rows(0xC0FFEE + nd, nd, 1000, 1000 + n, sigma)
    got = red.reduce_values(rows, nd)
    want, ok = _exact_reference(rows, nd)
    assert ok.mean() > 0.99
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))


def test_closed_form_power_of_two_is_exact_mean():
    rows = gen.grad_rows(11, 64, 0, 5000, 1e-3)
    got = red.reduce_values(rows, 64)
    exact = rows.view(np.float16).astype(np.float64).sum(axis=0) / 64.0
    assert np.array_equal(got.astype(np.float64), exact)


def test_hand_worked_cases(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "reduce_order_cases.json")))
    for c in d["cases"]:
        nd = c["nd"]
        rows = np.array([int(x, 16) for x in c["rows_f16"]], dtype=np.uint16).reshape(nd, 1)
        g32 = np.full(1, np.nan, dtype=np.float32)
        g16 = np.full(1, 0x7E00, dtype=np.uint16)
        # one-element shard: psi = nd, rank 0 owns [0, 1); the bucket is [0, 1)
        red.reduce_shard(nd, nd, 0, 0, 1, rows, g32, g16)
        assert hex(int(g32.view(np.uint32)[0])) == hex(int(c["grad32"], 16)), c["name"]
        assert hex(int(g16[0])) == hex(int(c["grad16"], 16)), c["name"]


def _rn32_of_reciprocal(nd):
    """The fp32 value nearest 1/nd by exact rational comparison (ties to even)."""
    from fractions import Fraction
    exact = Fraction(1, nd)
    f = np.float32(1.0 / nd)
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(1))]
    best = min(abs(Fraction(float(c)) - exact) for c in cands)
    near = [c for c in cands if abs(Fraction(float(c)) - exact) == best]
    return min(near, key=lambda c: int(c.view(np.uint32)) & 1)


def test_inv_nd_is_the_correctly_rounded_reciprocal():
    rng = np.random.default_rng(24)
    nds = [1, 2, 3, 7, 64, 400, 1000, 4096, 12345, (1 << 24) - 1, 1 << 24] + \
        [int(x) for x in rng.integers(1, 1 << 24, size=3000)]
    for nd in nds:
        assert red.inv_nd(nd).view(np.uint32) == _rn32_of_reciprocal(nd).view(np.uint32), nd


@pytest.mark.parametrize("nd", [0, (1 << 24) + 1, 1 << 30])
def test_inv_nd_refuses_nd_outside_the_exact_range(nd):
    with pytest.raises(ValueError):
        red.inv_nd(nd)


def test_nd1_is_identity():
    rows = gen.grad_rows(5, 1, 0, 10000, 0.3)
    got = red.reduce_values(rows, 1)
    assert np.array_equal(got, rows[0].view(np.float16).astype(np.float32))


@pytest.mark.parametrize("psi,nd,bucket", [(37, 3, 10), (100, 4, 7), (64, 8, 64), (13, 5, 3),
                                           (50, 1, 11)])
def test_brute_force_all_ranks(psi, nd, bucket):
    rows_full = gen.grad_rows(99, nd, 0, psi, 0.02)
    want = red.reduce_values(rows_full, nd)
    hi = psi
    buckets = []
    while hi > 0:                      # reverse order, as backward produces them
        lo = max(0, hi - bucket)
        buckets.append((lo, hi - lo))
        hi = lo
    flat = np.full(psi, np.nan, dtype=np.float32)
    for r in range(nd):
        s_lo, s_hi = geo.shard_range(psi, nd, r)
        g = np.full(s_hi - s_lo, np.nan, dtype=np.float32)
        written = np.zeros(s_hi - s_lo, dtype=np.int64)
        for off, n in buckets:
            before = g.copy()
            # the rows of this bucket are the local gradients of every rank
            a, b = red.reduce_shard(psi, nd, r, off, n, rows_full[:, off:off + n], g)
            changed = np.flatnonzero(~(np.isnan(before) & np.isnan(g)) & (before != g))
            assert np.all((changed + s_lo >= a) & (changed + s_lo < b))
            written[a - s_lo:b - s_lo] += 1
        assert np.all(written == 1)
        flat[s_lo:s_hi] = g
    assert np.array_equal(flat.view(np.uint32), want.view(np.uint32))


def test_outside_intersection_untouched():
    psi, nd, r = 100, 4, 1                 # shard [25, 50)
    rows = gen.grad_rows(3, nd, 40, 60, 0.1)
    g = np.full(25, -7.0, dtype=np.float32)
    a, b = red.reduce_shard(psi, nd, r, 40, 20, rows, g)
    assert (a, b) == (40, 50)
    assert np.all(g[:15] == -7.0)
    assert np.array_equal(g[15:], red.reduce_values(rows[:, :10], nd))


def test_empty_intersection_is_noop():
    g = np.full(25, 1.5, dtype=np.float32)
    rows = gen.grad_rows(3, 4, 0, 10, 0.1)
    assert red.reduce_shard(100, 4, 1, 0, 10, rows, g) == (25, 25)
    assert np.all(g == 1.5)


def test_bucket_beyond_psi_rejected():
    g = np.zeros(25, dtype=np.float32)
    with pytest.raises(ValueError):
        red.reduce_shard(100, 4, 1, 95, 10, np.zeros((4, 10), np.uint16), g)
