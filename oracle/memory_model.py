"""Per-device model-state memory of plain DP and the three ZeRO-DP stages.

Source: upskillscore guide "ZeRO: particionar estados do treino entre GPUs",
section "Como funciona".  Mixed-precision Adam keeps, for Psi parameters, 2 Psi
bytes of fp16 parameters, 2 Psi bytes of fp16 gradients and K Psi bytes of
optimizer state (fp32 master copy, momentum, variance; K = 12), 16 Psi in all.
Plain data parallelism replicates all of it on every device.  Stage 1 (P_os)
splits the optimizer state over the Nd data-parallel processes: 4 Psi +
K Psi / Nd.  Stage 2 (P_os+g) also keeps only the owned gradient partition.
Stage 3 (P_os+g+p) also partitions the parameters: 16 Psi / Nd.

Reading for stage 2: the guide gives only "about 2 Psi"; the exact bytes are
fp16 parameters (2 Psi) plus an fp16 gradient shard and the optimizer shard,
2 Psi + (2 + K) Psi / Nd, the one form that reproduces the guide's worked
figure of 16.6 GB for 7.5B parameters at Nd = 64 (section "Na pratica").

The guide writes the optimizer state as K Psi with K = 12 for mixed-precision
Adam; `k` keeps that multiplier general (the stage formulas are the same with
12 replaced by K: (4 + K) Psi, 4 Psi + K Psi / Nd, 2 Psi + (2 + K) Psi / Nd,
(4 + K) Psi / Nd).

Pins (tests/test_oracle_memory_model.py): the printed 120 / 31.4 / 16.6 / 1.9 GB
(tests/golden/memory_model_7p5b_nd64.json), the 16 Psi total, the limits of
4x and 8x as Nd grows, and 16 Psi / Nd linear in Nd; for general K, the limits
(4 + K) / 4 and (4 + K) / 2 and a brute-force sum over the bytes each stage
keeps per parameter.
"""
from __future__ import annotations

K_ADAM = 12          # optimizer-state bytes per parameter (fp32 copy, m, v)
FP16_BYTES = 2

STAGE_DP = 0
STAGE_OS = 1
STAGE_OS_G = 2
STAGE_OS_G_P = 3


def bytes_per_device(psi: float, nd: int, stage: int, k: int = K_ADAM) -> float:
    """Model-state bytes held by one data-parallel device."""
    if nd < 1:
        raise ValueError("nd must be >= 1")
    p = FP16_BYTES * psi      # fp16 parameters
    g = FP16_BYTES * psi      # fp16 gradients
    o = k * psi               # optimizer states
    if stage == STAGE_DP:
        return p + g + o
    if stage == STAGE_OS:
        return p + g + o / nd
    if stage == STAGE_OS_G:
        return p + (g + o) / nd
    if stage == STAGE_OS_G_P:
        return (p + g + o) / nd
    raise ValueError("stage must be 0 (DP), 1, 2 or 3")
