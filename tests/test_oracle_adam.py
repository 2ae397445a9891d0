"""Pins of oracle.adam.

* An fp64 transcription of Adam as published (Kingma & Ba, Algorithm 1:
  bias-corrected moments, epsilon outside the square root), written here
  separately from the oracle.  Per step, from the same fp32 input state, the
  oracle's fp32 results must agree within 8 fp32 ulps of each quantity's term
  scale (master |th| + |dth|, m b1|m| + c1|g|, v b2 v + c2 g^2); measured
  worst cases are about 4 ulps.
* The closed form with zero initial moments and a constant gradient:
  th_t = th_0 - t lr g / (|g| + eps) in real arithmetic.
* Special cases: a zero gradient from zero moments leaves the master weight
  unchanged and the moments +0.
* The per-step scalars against exact rational arithmetic.
* Sharded equals unsharded (lastdictionary entry "ZeRO", usage note: ZeRO
  changes where the state lives, not how updates are computed; llm-engineer
  card "ZeRO-2": each GPU updates only its shard and the all-gather rebuilds
  [A, B, C]): over all ranks of tiny models, the concatenated shard updates
  and the rebuilt fp16 vector equal one unsharded step; nothing outside a
  rank's fp16 slot is written.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import adam
from oracle import geometry as geo
from synth import gen

ULP = 2.0 ** -23


def textbook(th, m, v, g, lr, beta1, beta2, eps, t):
    """Adam, Algorithm 1 of Kingma & Ba, in fp64 on fp64 copies."""
    th, m, v, g = (np.asarray(x, dtype=np.float64) for x in (th, m, v, g))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    th = th - lr * m_hat / (np.sqrt(v_hat) + eps)
    return th, m, v


def _state(seed, n, sm, sv, sg, heavy=False):
    idx = np.arange(n, dtype=np.uint64)
    th = gen.state_f32(seed, gen.KIND_MASTER, idx, 0.02)
    m = gen.state_f32(seed, gen.KIND_M, idx, sm)
    v = gen.state_f32(seed, gen.KIND_V, idx, sv, absolute=True)
    g = gen.grad_f16(seed, 0, idx, sg, heavy_tail=heavy).view(np.float16).astype(np.float32)
    return th, m, v, g


def _within(got, want, scale, ulps):
    err = np.abs(got.astype(np.float64) - want)
    scale = np.asarray(scale, dtype=np.float64)
    return np.all(err <= ulps * ULP * scale), float((err / (ULP * scale + 1e-300)).max())


@pytest.mark.parametrize("case", [
    # (m sigma, v sigma, g sigma, lr, heavy tails)
    (1e-4, 1e-6, 1e-3, 1e-4, False),     # plain DP 1.4B-like state
    (0.0, 0.0, 5e-3, 1e-3, False),       # tiny ZeRO-2 rank: zero moments
    (0.0, 0.0, 1e-3, 1e-4, True),        # heavy-tailed gradients with exact zeros
])
def test_against_fp64_textbook(case):
    sm, sv, sg, lr, heavy = case
    th, m, v, g = _state(7, 50_000, sm, sv, sg, heavy)
    for t in range(1, 21):
        sc = adam.scalars(lr, 0.9, 0.999, 1e-8, t)
        th2, m2, v2, p16 = adam.step_values(th, m, v, g, sc)
        wth, wm, wv = textbook(th, m, v, g, lr, 0.9, 0.999, 1e-8, t)
        ok, e = _within(th2, wth, np.abs(th) + np.abs(wth - th), 8)
        assert ok, ("master", t, e)
        ok, e = _within(m2, wm, 0.9 * np.abs(m) + 0.1 * np.abs(g), 8)
        assert ok, ("m", t, e)
        ok, e = _within(v2, wv, 0.999 * v + 0.001 * g.astype(np.float64) ** 2, 8)
        assert ok, ("v", t, e)
        th, m, v = th2, m2, v2


def test_closed_form_constant_gradient():
    n = 50_000
    idx = np.arange(n, dtype=np.uint64)
    th0 = gen.state_f32(3, gen.KIND_MASTER, idx, 0.02)
    g = gen.grad_f16(3, 0, idx, 0.01).view(np.float16).astype(np.float32)
    g = g[g != 0]
    th0 = th0[:g.shape[0]]
    th, m, v = th0.copy(), np.zeros_like(g), np.zeros_like(g)
    lr = 1e-3
    g64 = g.astype(np.float64)
    for t in range(1, 4):
        th, m, v, _ = adam.step_values(th, m, v, g, adam.scalars(lr, 0.9, 0.999, 1e-8, t))
        want = th0.astype(np.float64) - t * lr * g64 / (np.abs(g64) + 1e-8)
        assert np.max(np.abs(th - want)) <= 1e-5 * t * lr
    # at t = 1 the textbook bound |dth| <= lr holds
    th1, _, _, _ = adam.step_values(th0, np.zeros_like(g), np.zeros_like(g), g,
                                    adam.scalars(lr, 0.9, 0.999, 1e-8, 1))
    assert np.all(np.abs(th1.astype(np.float64) - th0) <= lr * (1 + 1e-5))


def test_zero_gradient_from_zero_moments():
    th = gen.state_f32(4, gen.KIND_MASTER, np.arange(1000, dtype=np.uint64), 0.02)
    z = np.zeros(1000, np.float32)
    for t in (1, 2, 10):
        th2, m2, v2, p16 = adam.step_values(th, z, z, z, adam.scalars(1e-3, 0.9, 0.999, 1e-8, t))
        assert np.array_equal(th2.view(np.uint32), th.view(np.uint32))
        assert np.all(m2.view(np.uint32) == 0) and np.all(v2.view(np.uint32) == 0)
        assert np.array_equal(p16, th.astype(np.float16).view(np.uint16))


def test_fp16_gradient_widens_exactly():
    idx = np.arange(10_000, dtype=np.uint64)
    g16 = gen.grad_f16(5, 0, idx, 1e-3)
    th = gen.state_f32(5, gen.KIND_MASTER, idx, 0.02)
    m = gen.state_f32(5, gen.KIND_M, idx, 1e-4)
    v = gen.state_f32(5, gen.KIND_V, idx, 1e-6, absolute=True)
    sc = adam.scalars(1e-4, 0.9, 0.999, 1e-8, 3)
    a = adam.step_values(th, m, v, g16, sc)
    b = adam.step_values(th, m, v, g16.view(np.float16).astype(np.float32), sc)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _ulp32(x: Fraction) -> Fraction:
    f = abs(float(x))
    e = int(np.frexp(np.float32(f))[1]) - 24
    return Fraction(2) ** e


@pytest.mark.parametrize("lr,b1,b2,eps", [(1e-3, 0.9, 0.999, 1e-8), (1e-4, 0.9, 0.999, 1e-8),
                                          (3e-4, 0.8, 0.95, 1e-6)])
@pytest.mark.parametrize("t", [1, 2, 3, 10, 20, 1000])
def test_scalars_against_exact(lr, b1, b2, eps, t):
    sc = adam.scalars(lr, b1, b2, eps, t)
    L, B1, B2, E = (Fraction(str(x)) for x in (lr, b1, b2, eps))
    exact = {
        "b1": B1, "b2": B2, "c1": 1 - B1, "c2": 1 - B2, "eps": E,
        "step": L / (1 - B1 ** t),
    }
    for name, val in exact.items():
        got = Fraction(float(getattr(sc, name)))
        assert abs(got - val) <= _ulp32(val) / 2 * (1 + Fraction(1, 1000)), name
    # isb = 1 / sqrt(1 - beta2^t): check isb^2 * (1 - beta2^t) = 1 within 1 ulp each way
    bc2 = 1 - B2 ** t
    isb = Fraction(float(sc.isb))
    u = _ulp32(isb)
    assert (isb - u) ** 2 * bc2 < 1 < (isb + u) ** 2 * bc2


def test_scalars_reject_step_zero():
    with pytest.raises(ValueError):
        adam.scalars(1e-3, 0.9, 0.999, 1e-8, 0)


@pytest.mark.parametrize("psi,nd", [(1000, 3), (1 << 12, 4), (37, 5), (64, 1), (10, 16)])
def test_sharded_equals_unsharded(psi, nd):
    idx = np.arange(psi, dtype=np.uint64)
    th = gen.state_f32(9, gen.KIND_MASTER, idx, 0.02)
    m = gen.state_f32(9, gen.KIND_M, idx, 1e-4)
    v = gen.state_f32(9, gen.KIND_V, idx, 1e-6, absolute=True)
    g = gen.grad_f16(9, 0, idx, 1e-3).view(np.float16).astype(np.float32)
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    canary = np.uint16(0x7E01)
    for t in (1, 2, 3):
        # unsharded: one rank owns everything
        U = [th.copy(), m.copy(), v.copy()]
        flat_u = np.full(psi, canary, np.uint16)
        adam.adam_step_shard(psi, 1, 0, *U, g, flat_u, 0, t=t, **hp)
        # sharded: every rank updates its own shard and writes its slot
        S = [np.empty_like(th), np.empty_like(m), np.empty_like(v)]
        flat_s = np.full(psi, canary, np.uint16)
        for r in range(nd):
            lo, hi = geo.shard_range(psi, nd, r)
            sl = [th[lo:hi].copy(), m[lo:hi].copy(), v[lo:hi].copy()]
            before = flat_s.copy()
            adam.adam_step_shard(psi, nd, r, *sl, g[lo:hi], flat_s, 0, t=t, **hp)
            outside = np.ones(psi, bool)
            outside[lo:hi] = False
            assert np.array_equal(flat_s[outside], before[outside])
            for dst, src in zip(S, sl):
                dst[lo:hi] = src
        for a, b in zip(U, S):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(flat_u, flat_s)
        th, m, v = U


def test_slot_in_a_window():
    psi, nd, r = 100, 4, 2                      # shard [50, 75)
    n = 25
    th = np.linspace(-1, 1, n, dtype=np.float32)
    z = np.zeros(n, np.float32)
    g = np.full(n, 0.5, np.float32)
    win = np.full(40, 0x1234, np.uint16)        # window of flat [45, 85)
    adam.adam_step_shard(psi, nd, r, th, z.copy(), z.copy(), g, win, 45, 1e-3, 0.9, 0.999,
                         1e-8, 1)
    assert np.all(win[:5] == 0x1234) and np.all(win[30:] == 0x1234)
    assert np.array_equal(win[5:30], th.astype(np.float16).view(np.uint16))
    with pytest.raises(ValueError):
        adam.adam_step_shard(psi, nd, r, th, z.copy(), z.copy(), g, win, 51, 1e-3, 0.9, 0.999,
                             1e-8, 1)
