"""The owner's slice of the gradient reduce-scatter, one bucket at a time.

Sources:
* upskillscore guide, section "Como funciona": in stage 2 (P_os+g) each gradient
  is reduced only at the process that owns its partition, via reduce-scatter,
  and then released.
* llm-engineer card "ZeRO-2", section "Gradient lifecycle": as soon as a layer's
  or bucket's gradient is ready in backward it is reduce-scattered; the rank
  keeps only its own reduced shard and releases the rest of the local gradient.
  Section "ZeRO-1's remaining waste": rank k's local gradient is the full
  vector [g_k_A, g_k_B, g_k_C].

One GPU stands in for all Nd ranks: the Nd local fp16 gradients of a bucket
arrive as Nd rows, row k being rank k's local gradient over the bucket's flat
range.  The owner of shard [lo, hi) computes, for each flat index i in
bucket intersect shard:

    grad32[i - lo] = RN32( RN32(...RN32(RN32(+0 + x_0) + x_1)... + x_{Nd-1}) * inv )

with x_k = fp32(row_k[i]) (exact), additions in ascending rank order, each
rounded to fp32, and inv = RN32(1 / Nd) -- the data-parallel mean.  Readings
where the pages are silent: the summation order (ascending rank, starting from
+0), the scale (one fp32 multiply by the correctly rounded 1/Nd after the sum),
and the optional fp16 copy (grad16 = round-to-nearest-even of grad32).  Indices
outside the intersection are left untouched.

Pins (tests/test_oracle_reduce.py): a closed form -- fp16 values are integer
multiples of 2^-24, so while partial sums stay below 1 in magnitude the fp32
sum is exact and the result equals RN32(exact integer sum * inv); hand-worked
cases where the order of additions changes the bits
(tests/golden/reduce_order_cases.json); brute force over all ranks of a tiny
model (the union of the shards is the full mean gradient, nothing outside a
shard is written).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import geometry


MAX_ND = 1 << 24


def inv_nd(nd: int) -> np.float32:
    """RN32(1 / Nd): IEEE single division is correctly rounded, and fp32(Nd) is
    Nd itself for Nd <= 2^24; larger Nd are refused."""
    if not 1 <= nd <= MAX_ND:
        raise ValueError(f"Nd must lie in [1, 2^24], got {nd}")
    return np.float32(1.0) / np.float32(nd)


def reduce_values(rows: np.ndarray, nd: int) -> np.ndarray:
    """Mean over the Nd rows of fp16 bit patterns (uint16 [Nd, n]) -> fp32 [n]."""
    rows = np.asarray(rows)
    if rows.shape[0] != nd:
        raise ValueError("need exactly Nd rows")
    acc = np.zeros(rows.shape[1], dtype=np.float32)          # +0.0
    for k in range(nd):                                      # ascending rank order
        acc = acc + rows[k].view(np.float16).astype(np.float32)
    return acc * inv_nd(nd)


def reduce_shard(psi: int, nd: int, rank: int, bucket_offset: int, bucket_len: int,
                 rows: np.ndarray, grad32: np.ndarray,
                 grad16: Optional[np.ndarray] = None) -> Tuple[int, int]:
    """Reduce one bucket into the rank's shard-local gradient arrays, in place.

    rows: uint16 [Nd, >= bucket_len]; column j holds flat index bucket_offset + j.
    grad32: float32 [shard length]; grad16: optional uint16 [shard length].
    Returns the flat intersection [a, b) that was written.
    """
    lo, hi = geometry.shard_range(psi, nd, rank)
    if bucket_offset + bucket_len > psi:
        raise ValueError("bucket beyond the parameter vector")
    a, b = geometry.intersect(lo, hi, bucket_offset, bucket_len)
    if a == b:
        return a, b
    cols = rows[:, a - bucket_offset:b - bucket_offset]
    g = reduce_values(cols, nd)
    grad32[a - lo:b - lo] = g
    if grad16 is not None:
        grad16[a - lo:b - lo] = g.astype(np.float16).view(np.uint16)
    return a, b
