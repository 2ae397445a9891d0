"""Helpers of the GPU parity tests: device inputs from the shared generator,
sampling, and the comparison bars.

Bars (written here once, used by every parity test):
* reduce: bit-exact (fp32 and fp16 bits).
* Adam, per step from the same input state: master, m and v within 1e-6
  relative to max(|oracle|, term scale) -- term scales |th| + |dth|,
  b1 |m| + c1 |g|, b2 v + c2 g^2 -- and the fp16 parameter within 1 ulp.  The
  kernel performs the oracle's operations in the oracle's order with the same
  roundings, so the tests also assert bit equality.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from synth import device as sdev
from synth import gen

REL_TOL = 1e-6


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def gather(t: torch.Tensor, idx: np.ndarray) -> torch.Tensor:
    i = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int64)).to(t.device)
    return t.index_select(0, i)


def state_device(seed, lo, n, dist, kind, dev="cuda"):
    t = torch.empty(n, dtype=torch.float32, device=dev)
    sdev.fill_state(t, seed, kind, lo, dist.sigma, dist.absolute)
    return t


def state_host(seed, idx, dist, kind):
    return gen.state_f32(seed, kind, idx, dist.sigma, dist.absolute)


def rows_device(seed, nd, lo, n, dist, stride=None, dev="cuda"):
    stride = stride or n
    buf = torch.empty(nd * stride, dtype=torch.int16, device=dev)
    view = buf.as_strided((nd, n), (stride, 1))
    sdev.fill_grad_rows(view, seed, lo, dist.sigma, dist.heavy_tail)
    return view


def assert_bits(got: np.ndarray, want: np.ndarray, what: str):
    g = np.ascontiguousarray(got)
    w = np.ascontiguousarray(want)
    assert g.shape == w.shape, what
    gb = g.view(np.uint32 if g.dtype.itemsize == 4 else np.uint16)
    wb = w.view(np.uint32 if w.dtype.itemsize == 4 else np.uint16)
    bad = np.flatnonzero(gb != wb)
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:5]}: "
                           f"got {g.ravel()[bad[:5]]} want {w.ravel()[bad[:5]]}")


def _ordered16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def assert_adam_step(prev, got, want, c1=0.1, b1=0.9, b2=0.999, c2=0.001, what=""):
    """prev = (th, m, v, g) inputs of the step; got/want = (th, m, v, p16)."""
    th0, m0, v0, g0 = (np.asarray(x, np.float64) for x in prev)
    gth, gm, gv, gp = got
    wth, wm, wv, wp = want
    dth = np.abs(wth.astype(np.float64) - th0)
    scales = (np.abs(th0) + dth, b1 * np.abs(m0) + c1 * np.abs(g0), b2 * v0 + c2 * g0 * g0)
    for name, x, y, sc in (("master", gth, wth, scales[0]), ("m", gm, wm, scales[1]),
                           ("v", gv, wv, scales[2])):
        ref = np.maximum(np.abs(y.astype(np.float64)), sc)
        err = np.abs(x.astype(np.float64) - y.astype(np.float64))
        worst = float(np.max(err / np.maximum(ref, 1e-300))) if err.size else 0.0
        assert np.all(err <= REL_TOL * ref), f"{what} {name}: relative error {worst:.3g} > 1e-6"
    d16 = np.abs(_ordered16(gp) - _ordered16(wp))
    assert np.all(d16 <= 1), f"{what} p16: {int(d16.max())} ulp"
    for name, x, y in (("master", gth, wth), ("m", gm, wm), ("v", gv, wv), ("p16", gp, wp)):
        assert_bits(x, y, f"{what} {name} bits")


def sample_indices(n: int, edges, count: int, seed: int) -> np.ndarray:
    """Shard-local sample: every edge +-64 (clipped), plus `count` random picks."""
    rng = np.random.default_rng(seed)
    pts = [np.arange(0, min(n, 64)), np.arange(max(0, n - 64), n)]
    for e in edges:
        pts.append(np.arange(max(0, e - 64), min(n, e + 64)))
    pts.append(rng.integers(0, n, size=count))
    return np.unique(np.concatenate(pts)).astype(np.int64)
