"""Two device properties through the C ABI, against the oracle.

* The fp16 parameter slot rounds every fp32 value exactly as the oracle does
  (IEEE round-to-nearest-even; the oracle's conversion is pinned to an integer
  implementation of the standard in tests/test_fp16_rounding.py).  With zero
  moments and a zero gradient the Adam step leaves the master weight unchanged
  (th - step * (0 / eps) = th), so the slot it writes is the conversion of the
  input itself: every fp16 value, the fp32 midpoints between neighbouring fp16
  values and their fp32 neighbours, the fp16 subnormal and overflow edges,
  random patterns over all exponents, and the special values.
* Stopping after k steps, copying the state (master, m, v and the step count)
  to the host and back into fresh buffers, and continuing, gives the same bits
  as running straight through -- the state of the path is exactly
  (master, m, v, t).
"""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_bucketed_amd as Z
from gpu_util import assert_bits, f32, need_gpu, u16
from synth import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


def _conversion_inputs() -> np.ndarray:
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = h[(h & 0x7C00) != 0x7C00]
    v = finite.view(np.float16).astype(np.float32)
    with np.errstate(over="ignore"):
        nxt = np.nextafter(finite.view(np.float16), np.float16(np.inf)).astype(np.float32)
    ok = np.isfinite(nxt)
    mid = ((v[ok].astype(np.float64) + nxt[ok].astype(np.float64)) / 2).astype(np.float32)
    pts = [v, mid]
    for d in (1, 2, 3):                                       # fp32 neighbours of the midpoints
        pts.append(np.nextafter(mid, np.float32(np.inf)))
        pts.append(np.nextafter(mid, np.float32(-np.inf)))
        mid = np.nextafter(mid, np.float32(np.inf))
    edges = np.array([65504.0, 65519.99, 65520.0, 65520.01, 1e5, 3.4e38, 2.0 ** -24, 2.0 ** -25,
                      2.0 ** -25 * 1.0000001, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * 0.9999999,
                      1e-45, 0.0], dtype=np.float32)
    pts += [edges, -edges]
    rng = np.random.default_rng(2024)
    pts.append(rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
               .view(np.float32))
    specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                         0x7FBFFFFF, 0x80000000, 0x00000001, 0x807FFFFF], np.uint32).view(np.float32)
    pts.append(specials)
    return np.concatenate(pts).astype(np.float32)


def test_fp16_slot_rounding_matches_oracle():
    th = _conversion_inputs()
    n = th.size
    print(f"conversion cases: {n}", flush=True)
    geom = Z.shard_geometry(n, 1, 0)
    d_th = torch.from_numpy(th.copy()).cuda()
    zeros = torch.zeros(n, dtype=torch.float32, device="cuda")
    m, v, g = zeros.clone(), zeros.clone(), zeros.clone()
    p16 = torch.zeros(n, dtype=torch.int16, device="cuda")
    Z.adam_step_shard(geom, d_th, m, v, g, p16, 0, 1e-3, 0.9, 0.999, 1e-8, 1)
    torch.cuda.synchronize()
    got_th, got_p = f32(d_th), u16(p16)
    with np.errstate(all="ignore"):
        want_p = th.astype(np.float16).view(np.uint16)         # the oracle's conversion
    nan = np.isnan(th)
    assert_bits(got_th[~nan], th[~nan], "master unchanged by a zero step")
    assert np.all(np.isnan(got_th[nan]))
    assert_bits(got_p[~nan], want_p[~nan], "fp16 slot")
    assert np.all((got_p[nan] & 0x7C00) == 0x7C00) and np.all((got_p[nan] & 0x03FF) != 0)


@pytest.mark.parametrize("g16", [False, True])
def test_resume_from_saved_state_is_bit_identical(g16):
    psi, nd, rank, k, j = 2_000_003, 3, 1, 3, 4
    geom = Z.shard_geometry(psi, nd, rank)
    lo, n = geom.offset, geom.len
    idx = np.arange(lo, lo + n, dtype=np.uint64)
    th0 = gen.state_f32(11, gen.KIND_MASTER, idx, 0.02)
    m0 = gen.state_f32(11, gen.KIND_M, idx, 1e-4)
    v0 = gen.state_f32(11, gen.KIND_V, idx, 1e-6, True)
    gb = gen.grad_f16(11, 0, idx, 1e-3)
    grad = torch.from_numpy(gb.view(np.int16) if g16 else gb.view(np.float16).astype(np.float32)) \
        .cuda()

    def fresh(state):
        return [torch.from_numpy(a.copy()).cuda() for a in state]

    def steps(state, t0, t1, flat16):
        for t in range(t0, t1 + 1):
            Z.adam_step_shard(geom, *state, grad, flat16, 0, 1e-4, 0.9, 0.999, 1e-8, t)

    straight = fresh((th0, m0, v0))
    flat_a = torch.zeros(psi, dtype=torch.int16, device="cuda")
    steps(straight, 1, k + j, flat_a)
    first = fresh((th0, m0, v0))
    flat_b = torch.zeros(psi, dtype=torch.int16, device="cuda")
    steps(first, 1, k, flat_b)
    torch.cuda.synchronize()
    saved = {"master": f32(first[0]).copy(), "m": f32(first[1]).copy(), "v": f32(first[2]).copy(),
             "t": k}
    del first
    resumed = fresh((saved["master"], saved["m"], saved["v"]))
    steps(resumed, saved["t"] + 1, k + j, flat_b)
    torch.cuda.synchronize()
    for a, b, name in zip(straight, resumed, ("master", "m", "v")):
        assert_bits(f32(b), f32(a), f"resumed {name}")
    assert_bits(u16(flat_b), u16(flat_a), "fp16 vector")
