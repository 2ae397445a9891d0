"""Seeded synthetic inputs, host side (NumPy).

This module generates the inputs of the per-rank ZeRO path: the Nd local
fp16 gradient rows of a bucket and the fp32 master / momentum / variance
shards.  It holds none of the method's arithmetic (no reduction, no optimizer
update); both the CPU oracle and the GPU path take their inputs from here, and
``synth/csrc/synth_gen.hip`` is a second implementation of the same generator
definition for device-side generation at full size.

Generator definition (shared by both implementations, bit for bit):

* ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; constants of
  Stafford's variant 13 as used in the reference splitmix64.c):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
* A stream is keyed by (seed, kind, rank):
  ``key = mix64(seed ^ (kind << 56) ^ rank)``.
* Element ``i`` (a flat parameter index) of a stream draws
  ``x = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``.
* Normal values come from a 2**16-entry quantile table indexed by the top 16
  bits of ``x``: ``T[j] = round(sigma * Phi^-1((j + 0.5) / 2**16))`` computed in
  fp64 and rounded once (round-to-nearest-even) to the target dtype.  No
  transcendental function runs on the device, so both sides agree exactly.
* Heavy-tailed gradients use bits 32..47 of ``x`` as a uniform ``u`` in
  [0, 2**16): ``u < 655`` gives +0.0, ``u < 1311`` gives an outlier from the
  table of ``100 * sigma``, anything else the table of ``sigma``.
"""
from __future__ import annotations

import functools
import statistics

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream kinds.
KIND_GRAD = 1       # local fp16 gradient of data-parallel rank `rank`
KIND_MASTER = 2     # fp32 master weights
KIND_M = 3          # fp32 first moment
KIND_V = 4          # fp32 second moment
KIND_GRAD_FULL = 5  # fp16 gradient of a plain data-parallel (Nd = 1) run
KIND_PARAM16 = 6    # fp16 parameters held in a stage-3 rank shard

# Heavy-tail thresholds on the 16-bit uniform (about 1% zeros, 1% outliers).
TAIL_ZERO_BELOW = 655
TAIL_OUTLIER_BELOW = 1311
TAIL_SCALE = 100.0


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, kind: int, rank: int) -> int:
    """64-bit key of the stream (seed, kind, rank)."""
    if not (0 <= kind < 256 and 0 <= rank < (1 << 32)):
        raise ValueError("kind must fit 8 bits and rank 32 bits")
    return mix64_int((seed & MASK64) ^ (kind << 56) ^ rank)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def draws(key: int, index: np.ndarray) -> np.ndarray:
    """Raw 64-bit draws of a stream at the given flat indices (uint64)."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        return _mix64_np(z)


@functools.lru_cache(maxsize=None)
def _quantiles() -> np.ndarray:
    nd = statistics.NormalDist()
    return np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)],
                    dtype=np.float64)


@functools.lru_cache(maxsize=None)
def table_f16(sigma: float) -> np.ndarray:
    """2**16 fp16 normal quantiles of N(0, sigma), as uint16 bit patterns."""
    t = (_quantiles() * float(sigma)).astype(np.float16)
    t.setflags(write=False)
    return t.view(np.uint16)


@functools.lru_cache(maxsize=None)
def table_f32(sigma: float, absolute: bool = False) -> np.ndarray:
    """2**16 fp32 normal quantiles of N(0, sigma) (or |N(0, sigma)|)."""
    q = _quantiles() * float(sigma)
    if absolute:
        q = np.abs(q)
    t = q.astype(np.float32)
    t.setflags(write=False)
    return t


def grad_f16(seed: int, rank: int, index: np.ndarray, sigma: float,
             heavy_tail: bool = False, kind: int = KIND_GRAD) -> np.ndarray:
    """fp16 gradient values (uint16 bit patterns) of rank `rank` at `index`."""
    x = draws(stream_key(seed, kind, rank), index)
    j = (x >> np.uint64(48)).astype(np.intp)
    out = table_f16(sigma)[j]
    if heavy_tail:
        u = ((x >> np.uint64(32)) & np.uint64(0xFFFF)).astype(np.int64)
        out = np.where(u < TAIL_OUTLIER_BELOW,
                       table_f16(sigma * TAIL_SCALE)[j], out)
        out = np.where(u < TAIL_ZERO_BELOW, np.uint16(0), out)
    return out.astype(np.uint16)


def state_f32(seed: int, kind: int, index: np.ndarray, sigma: float,
              absolute: bool = False) -> np.ndarray:
    """fp32 state values (master, m or v) at `index`; sigma 0 gives zeros."""
    idx = np.asarray(index, dtype=np.uint64)
    if sigma == 0.0:
        return np.zeros(idx.shape, dtype=np.float32)
    x = draws(stream_key(seed, kind, 0), idx)
    return table_f32(sigma, absolute)[(x >> np.uint64(48)).astype(np.intp)]


def grad_rows(seed: int, nd: int, lo: int, hi: int, sigma: float,
              heavy_tail: bool = False) -> np.ndarray:
    """All Nd local gradient rows over the flat range [lo, hi): uint16 [nd, hi-lo]."""
    idx = np.arange(lo, hi, dtype=np.uint64)
    out = np.empty((nd, hi - lo), dtype=np.uint16)
    for k in range(nd):
        out[k] = grad_f16(seed, k, idx, sigma, heavy_tail)
    return out
