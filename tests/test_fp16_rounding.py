"""Pins of the fp16 conversions the oracle relies on (NumPy's casts) against
an integer implementation of the IEEE 754 definition (tests/fp16_exact.py)
and Python's own binary16 codec.

The fp16 widening feeds the reduce (every fp16 gradient widens exactly to
fp32); the fp32 -> fp16 round-to-nearest-even narrowing makes the fp16 copy of
the reduced gradient and the fp16 parameter slot that the all-gather would
distribute (llm-engineer card "ZeRO-2", "Why all-gather is still needed").
"""
import numpy as np

from fp16_exact import f16_bits_to_float, f32_bits_to_f16_bits


def test_widening_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    w = h.view(np.float16).astype(np.float32)
    for b in range(0, 1 << 16, 1):
        if (b & 0x7C00) == 0x7C00 and (b & 0x3FF):
            assert np.isnan(w[b])
            continue
        assert float(w[b]) == f16_bits_to_float(b)


def _check(bits32):
    bits32 = np.asarray(bits32, dtype=np.uint32)
    with np.errstate(over="ignore", invalid="ignore"):
        got = bits32.view(np.float32).astype(np.float16).view(np.uint16)
    for b, g in zip(bits32.tolist(), got.tolist()):
        want = f32_bits_to_f16_bits(b)
        if (want & 0x7C00) == 0x7C00 and (want & 0x3FF):
            assert (g & 0x7C00) == 0x7C00 and (g & 0x3FF), hex(b)   # NaN stays NaN
        else:
            assert g == want, (hex(b), hex(g), hex(want))


def test_narrowing_at_every_midpoint():
    # the exact midpoints between consecutive positive finite fp16 values, and
    # their fp32 neighbours, both signs -- every rounding decision of the cast
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    lo = pos.view(np.float16).astype(np.float64)
    hi = np.append(lo[1:], 65536.0)
    mid = ((lo + hi) / 2).astype(np.float32)            # exact in fp32 (12 significant bits)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    b = mid.view(np.uint32)
    cand = np.concatenate([b, b - 1, b + 1, lo.astype(np.float32).view(np.uint32)])
    cand = cand[cand < 0x7F800000]
    _check(np.concatenate([cand, cand | np.uint32(0x80000000)]))


def test_narrowing_random_and_special():
    rng = np.random.default_rng(1234)
    r = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x33000000, 0x33000001,
                        0x337FFFFF, 0x33800000, 0x477FE000, 0x477FEFFF, 0x477FF000,
                        0x477FF001, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000,
                        0x3F800000, 0x3F801000, 0x3F802000, 0x3F803000], dtype=np.uint32)
    _check(np.concatenate([r, special]))


def test_named_values():
    # 65504 is the largest finite fp16; 65520 is the tie with 65536 and rounds to inf
    assert f32_bits_to_f16_bits(int(np.float32(65504).view(np.uint32))) == 0x7BFF
    assert f32_bits_to_f16_bits(int(np.float32(65519.996).view(np.uint32))) == 0x7BFF
    assert f32_bits_to_f16_bits(int(np.float32(65520).view(np.uint32))) == 0x7C00
    # 2^-25 is the tie between 0 and the smallest subnormal 2^-24 -> 0 (even)
    assert f32_bits_to_f16_bits(0x33000000) == 0x0000
    assert f32_bits_to_f16_bits(0x33000001) == 0x0001
    # 1 + 2^-11 ties between 1 and 1 + 2^-10 -> 1 (even); 1 + 3*2^-11 -> 1 + 2^-9
    assert f32_bits_to_f16_bits(0x3F801000) == 0x3C00
    assert f32_bits_to_f16_bits(0x3F803000) == 0x3C02


def _binade_mismatches(args):
    import numpy as np
    from fp16_exact import f16_bits_of_binade
    sign, e = args
    bits = (np.uint32(sign << 31) | np.uint32(e << 23)) | np.arange(1 << 23, dtype=np.uint32)
    with np.errstate(over="ignore", invalid="ignore"):
        got = bits.view(np.float32).astype(np.float16).view(np.uint16)
    if e == 0xFF:                      # NaN stays NaN (payloads are not compared), inf exact
        want = f16_bits_of_binade(sign, e)
        nan = (want & 0x3FF) != 0
        bad = ((got & 0x7C00) != 0x7C00) | (((got & 0x3FF) != 0) != nan)
        return int(np.count_nonzero(bad | (~nan & (got != want))))
    lo = f32_bits_to_f16_bits(int(bits[0]))
    hi = f32_bits_to_f16_bits(int(bits[-1]))
    if lo == hi:
        # rounding is monotone within a binade: equal ends mean the whole binade
        # maps to that one value (all of +-0 below 2^-25, all of +-inf from 65536)
        return int(np.count_nonzero(got != lo))
    return int(np.count_nonzero(got != f16_bits_of_binade(sign, e)))


def test_narrowing_exhaustive_all_fp32():
    """NumPy's fp32 -> fp16 cast (the oracle's) against the integer definition on
    every one of the 2^32 fp32 bit patterns, one binade (sign, exponent) at a time."""
    import multiprocessing as mp
    import os
    import time
    jobs = [(s, e) for s in (0, 1) for e in range(256)]
    t0 = time.time()
    workers = max(1, min(4, len(os.sched_getaffinity(0))))
    with mp.get_context("fork").Pool(workers) as pool:
        bad = pool.map(_binade_mismatches, jobs, chunksize=8)
    assert sum(bad) == 0, [(j, b) for j, b in zip(jobs, bad) if b][:5]
    print(f"2^32 patterns checked in {time.time() - t0:.1f} s with {workers} processes")
