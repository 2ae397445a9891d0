"""The workloads of the per-rank ZeRO path: sizes, bucket schedules, seeds.

Each workload is one data-parallel rank of a model of ``psi`` parameters
trained with ``nd`` data-parallel ranks.  Sizes follow the models the pages
discuss (7.5B at Nd = 64 in the worked memory example, 1.4B where plain
PyTorch data parallelism runs out of memory, 13B trained without model
parallelism, 100B with hidden size 8192).  Gradient buckets are flat ranges of
the parameter vector that arrive in reverse layer order, as a backward pass
produces them (ZeRO-2 card, "Gradient lifecycle").

Nothing here computes any part of the method: bucket schedules and value
distributions are workload structure, shared by the oracle and the GPU path.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

BUCKET = 25_000_000          # uniform gradient bucket size (elements)
SEED_BASE = 0x5EED0000


@dataclass(frozen=True)
class Dist:
    """Value distribution: N(0, sigma) (or |N(0, sigma)|); sigma 0 means zeros."""
    sigma: float
    absolute: bool = False
    heavy_tail: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    psi: int
    nd: int
    rank: int
    buckets: Tuple[Tuple[int, int], ...]   # (flat offset, length) in arrival order
    grad: Dist
    master: Dist
    m: Dist
    v: Dist
    lr: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    steps: int = 1
    seed: int = SEED_BASE
    # Nd = 1 plain data parallelism: the optimizer reads the raw fp16 gradient
    # (no reduce, no fp32 gradient shard).
    fp16_grad: bool = False
    # ZeRO-2 gradient shard the reduce writes and Adam reads: "fp32", or "fp16"
    # (the 2-byte gradient shard of the guide's 2 Psi + 14 Psi / Nd accounting).
    grad_shard: str = "fp32"
    extra: dict = field(default_factory=dict, compare=False)


def uniform_buckets(psi: int, size: int = BUCKET) -> Tuple[Tuple[int, int], ...]:
    """Buckets cut from the end of the flat space; arrival order = highest first."""
    out: List[Tuple[int, int]] = []
    hi = psi
    while hi > 0:
        lo = max(0, hi - size)
        out.append((lo, hi - lo))
        hi = lo
    return tuple(out)


def transformer_tensors(psi: int, hidden: int) -> List[Tuple[int, int]]:
    """Flat (offset, length) of each tensor of a stack of transformer layers.

    Per layer, in forward order: attention 4h^2, MLP 8h^2, layer norms 2h.  Layers
    repeat until psi is reached; the last tensor is truncated so the total is psi.
    """
    sizes = (4 * hidden * hidden, 8 * hidden * hidden, 2 * hidden)
    out: List[Tuple[int, int]] = []
    off = 0
    while off < psi:
        for s in sizes:
            if off >= psi:
                break
            n = min(s, psi - off)
            out.append((off, n))
            off += n
    return out


def transformer_layers(psi: int, hidden: int) -> List[Tuple[int, int]]:
    """Flat (offset, length) of each layer (its three tensors together), forward order."""
    per = 12 * hidden * hidden + 2 * hidden
    return [(off, min(per, psi - off)) for off in range(0, psi, per)]


def tensor_buckets(psi: int, hidden: int, size: int = BUCKET) -> Tuple[Tuple[int, int], ...]:
    """Buckets = tensors in reverse order, each cut from its end into <= size pieces."""
    out: List[Tuple[int, int]] = []
    for off, n in reversed(transformer_tensors(psi, hidden)):
        hi = off + n
        while hi > off:
            lo = max(off, hi - size)
            out.append((lo, hi - lo))
            hi = lo
    return tuple(out)


def _c(i: int) -> int:
    return SEED_BASE + i


def tiny(psi: int = 1 << 20, nd: int = 4, rank: int = 0) -> Workload:
    """Tiny ZeRO-2 rank: psi = 2^20, Nd = 4, one bucket, 3 Adam steps."""
    return Workload(
        name=f"tiny-zero2-psi{psi}-nd{nd}-r{rank}", psi=psi, nd=nd, rank=rank,
        buckets=((0, psi),), grad=Dist(0.01), master=Dist(0.02), m=Dist(0.0),
        v=Dist(0.0), lr=1e-3, steps=3, seed=_c(0))


def plain_dp_1p4b(psi: int = 1_400_000_000) -> Workload:
    """Plain data parallelism (Nd = 1, no reduce) of a 1.4B model, fp16 grads."""
    return Workload(
        name=f"plain-dp-psi{psi}", psi=psi, nd=1, rank=0, buckets=(),
        grad=Dist(1e-3), master=Dist(0.02), m=Dist(1e-4),
        v=Dist(1e-6, absolute=True), lr=1e-4, steps=20, seed=_c(1),
        fp16_grad=True)


def zero2_7p5b(rank: int = 0) -> Workload:
    """ZeRO-2 rank of a 7.5B model at Nd = 64 (shard of 117,187,500)."""
    psi = 7_500_000_000
    return Workload(
        name=f"zero2-7.5B-nd64-r{rank}", psi=psi, nd=64, rank=rank,
        buckets=uniform_buckets(psi), grad=Dist(1e-3), master=Dist(0.02),
        m=Dist(1e-4), v=Dist(1e-6, absolute=True), lr=1e-4, steps=10,
        seed=_c(2))


def zero2_7p5b_g16(rank: int = 0) -> Workload:
    """The 7.5B / Nd = 64 rank with an fp16 gradient shard."""
    w = zero2_7p5b(rank)
    return Workload(**{**w.__dict__, "name": f"zero2-7.5B-nd64-g16-r{rank}",
                       "grad_shard": "fp16"})


def zero3_7p5b(rank: int = 0) -> Workload:
    """Stage-3 rank of the 7.5B model at Nd = 64: hidden 4096 (37 layers of
    12 h^2 + 2 h and a truncated last one), each layer's parameters gathered in
    forward and in backward, the layer gradients reduced per layer, an fp16
    gradient shard."""
    w = zero2_7p5b(rank)
    return Workload(**{**w.__dict__, "name": f"zero3-7.5B-nd64-r{rank}",
                       "buckets": tuple(reversed(transformer_layers(w.psi, 4096))),
                       "grad_shard": "fp16",
                       "extra": {"stage": 3, "hidden": 4096, "param_sigma": 0.02}})


def zero2_13b(rank: int = 0) -> Workload:
    """ZeRO-2 rank of a 13B model at Nd = 32 with heavy-tailed gradients."""
    psi = 13_000_000_000
    return Workload(
        name=f"zero2-13B-nd32-r{rank}", psi=psi, nd=32, rank=rank,
        buckets=uniform_buckets(psi), grad=Dist(1e-3, heavy_tail=True),
        master=Dist(0.02), m=Dist(0.0), v=Dist(0.0), lr=1e-4, steps=10,
        seed=_c(3), extra={"probe": 1 << 20})


def zero2_100b(rank: int = 137) -> Workload:
    """ZeRO-2 rank 137 of a 100B model (hidden 8192) at Nd = 400."""
    psi = 100_000_000_000
    return Workload(
        name=f"zero2-100B-nd400-r{rank}", psi=psi, nd=400, rank=rank,
        buckets=tensor_buckets(psi, 8192), grad=Dist(1e-3), master=Dist(0.02),
        m=Dist(1e-4), v=Dist(1e-6, absolute=True), lr=1e-4, steps=5,
        seed=_c(4), extra={"chunk": 1 << 22, "p16_window": 1 << 20})


def buckets_touching(buckets, lo: int, hi: int):
    """Buckets (in arrival order) whose range meets [lo, hi)."""
    return [(o, n) for (o, n) in buckets if o < hi and o + n > lo]
