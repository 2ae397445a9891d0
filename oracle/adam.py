"""The sharded mixed-precision Adam step and the fp16 slot write.

Sources:
* upskillscore guide, section "Como funciona": mixed-precision Adam keeps an
  fp32 copy of the parameters, the momentum and the variance (K = 12 bytes per
  parameter); in stage 1 and 2 each process updates only its own partition of
  that state and an all-gather distributes the updated parameters.
* lastdictionary entry "ZeRO", usage note: ZeRO changes where optimizer state
  is stored, not how updates are computed -- so the sharded step is the plain
  Adam update restricted to the owned partition.
* llm-engineer card "ZeRO-2", sections "Gradient lifecycle" and "Why all-gather
  is still needed": each GPU updates only its parameter shard; the updated fp16
  shard goes to its place in the full parameter vector that the all-gather
  rebuilds as [updated A, updated B, updated C].

The pages do not print the Adam formula.  Reading: Adam as published by
Kingma & Ba (ICLR 2015, Algorithm 1) -- bias-corrected moments, epsilon added
to the square root of the corrected variance, step t counted from 1, no weight
decay, clipping or loss scaling (the pages mention none).  Written per element
in fp32, every operation rounded once (no fused multiply-add), with scalars
derived on the host in fp64 and rounded once to fp32:

    b1 = RN32(beta1)        c1 = RN32(1 - beta1)
    b2 = RN32(beta2)        c2 = RN32(1 - beta2)
    step = RN32(lr / (1 - beta1^t))      isb = RN32(1 / sqrt(1 - beta2^t))
    e = RN32(eps)

    m'  = b1*m + c1*g
    v'  = b2*v + c2*(g*g)
    den = sqrt(v')*isb + e
    th' = th - step*(m'/den)
    p16 = fp16 round-to-nearest-even of th'

In real arithmetic th' = th - lr * mhat / (sqrt(vhat) + eps) with
mhat = m'/(1 - beta1^t) and vhat = v'/(1 - beta2^t), i.e. Algorithm 1.  The fp32
operation order is a fixed reading, not something the pages fix.

Pins (tests/test_oracle_adam.py): an fp64 transcription of Algorithm 1 written
separately (per-step agreement within a few fp32 ulps of the term scale);
the closed form with m = v = 0 and a constant gradient (th_t = th_0 -
t*lr*g/(|g| + eps) in real arithmetic); special cases (zero gradient from zero
moments leaves th unchanged); and the sharded-equals-unsharded invariant over
all ranks of a tiny model, including the rebuilt fp16 vector.

Parity unpinned: the exact last bits of the step.  Where Algorithm 1 leaves the
fp32 operation order open they follow the fixed order above; the pins hold them
to within a few ulps of the term scale, not bit for bit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import geometry


@dataclass(frozen=True)
class Scalars:
    b1: np.float32
    b2: np.float32
    c1: np.float32
    c2: np.float32
    eps: np.float32
    step: np.float32
    isb: np.float32

    def as_tuple(self):
        return (self.b1, self.b2, self.c1, self.c2, self.eps, self.step, self.isb)


def scalars(lr: float, beta1: float, beta2: float, eps: float, t: int) -> Scalars:
    """Per-step fp32 scalars, derived in fp64 and rounded once."""
    if t < 1:
        raise ValueError("step t counts from 1")
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    return Scalars(
        b1=np.float32(beta1), b2=np.float32(beta2),
        c1=np.float32(1.0 - beta1), c2=np.float32(1.0 - beta2),
        eps=np.float32(eps),
        step=np.float32(lr / bc1),
        isb=np.float32(1.0 / math.sqrt(bc2)))


def grad_f32(grad: np.ndarray) -> np.ndarray:
    """The gradient as fp32: fp32 passes through, fp16 bit patterns widen exactly."""
    grad = np.asarray(grad)
    if grad.dtype == np.float32:
        return grad
    if grad.dtype == np.uint16:
        return grad.view(np.float16).astype(np.float32)
    if grad.dtype == np.float16:
        return grad.astype(np.float32)
    raise TypeError("gradient must be float32, float16 or uint16 fp16 bits")


def step_values(master, m, v, grad, sc: Scalars):
    """One Adam step on arrays; returns (master', m', v', p16 bits). Inputs untouched."""
    g = grad_f32(grad)
    m_new = sc.b1 * m + sc.c1 * g
    v_new = sc.b2 * v + sc.c2 * (g * g)
    den = np.sqrt(v_new) * sc.isb + sc.eps
    th = master - sc.step * (m_new / den)
    p16 = th.astype(np.float16).view(np.uint16)
    return th, m_new, v_new, p16


def adam_step_shard(psi: int, nd: int, rank: int, master: np.ndarray, m: np.ndarray,
                    v: np.ndarray, grad: np.ndarray, param16: Optional[np.ndarray],
                    param16_origin: int, lr: float, beta1: float, beta2: float,
                    eps: float, t: int) -> None:
    """Update the rank's shard in place and write its fp16 slot.

    master/m/v/grad cover the shard [lo, hi) (shard-local index).  param16 is a
    uint16 window of the flat fp16 parameter vector starting at flat index
    param16_origin; the slot [lo, hi) is written, nothing else.
    """
    lo, hi = geometry.shard_range(psi, nd, rank)
    n = hi - lo
    for a in (master, m, v, grad):
        if a.shape[0] != n:
            raise ValueError("state arrays must have the shard length")
    th, m_new, v_new, p16 = step_values(master, m, v, grad, scalars(lr, beta1, beta2, eps, t))
    master[...] = th
    m[...] = m_new
    v[...] = v_new
    if param16 is not None:
        if lo < param16_origin or hi - param16_origin > param16.shape[0]:
            raise ValueError("the fp16 window does not hold the shard's slot")
        param16[lo - param16_origin:hi - param16_origin] = p16
