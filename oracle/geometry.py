"""Shard geometry: which flat parameter range a data-parallel rank owns.

Source: llm-engineer card "ZeRO-2", sections "Gradient lifecycle" and "Why
all-gather is still needed": the flat parameter space is split into Nd
partitions (A, B, C for three GPUs), rank r owns partition r, and the
all-gather of the updated partitions, in rank order, rebuilds the full vector
[A, B, C].  So partitions are contiguous and rank-major.

Reading where the pages are silent: when Nd does not divide Psi, the shard
size is S = ceil(Psi / Nd) and trailing shards are short (possibly empty).

Pins (tests/test_oracle_geometry.py): brute force on tiny Psi -- the shards of
all ranks are disjoint, cover [0, Psi) exactly and concatenate in rank order.
"""
from __future__ import annotations

from typing import Tuple


def shard_size(psi: int, nd: int) -> int:
    if nd < 1:
        raise ValueError("nd must be >= 1")
    return -(-psi // nd)


def shard_range(psi: int, nd: int, rank: int) -> Tuple[int, int]:
    """Flat range [lo, hi) owned by `rank`."""
    if not 0 <= rank < nd:
        raise ValueError("rank out of range")
    s = shard_size(psi, nd)
    return min(rank * s, psi), min((rank + 1) * s, psi)


def intersect(lo: int, hi: int, off: int, n: int) -> Tuple[int, int]:
    """[lo, hi) intersected with [off, off + n); empty gives (x, x)."""
    a = max(lo, off)
    b = min(hi, off + n)
    return (a, b) if a < b else (a, a)
