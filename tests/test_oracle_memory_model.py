"""Pins of oracle.memory_model against what the pages fix.

upskillscore guide "ZeRO: particionar estados do treino entre GPUs":
section "Como funciona" (16 Psi accounting, K = 12, stage formulas, limits of
4x and 8x, linear in Nd for stage 3) and section "Na pratica" (the printed
7.5B / Nd = 64 figures).  lastdictionary entry "ZeRO" repeats the limits.
"""
import json
import os

import pytest

from oracle import memory_model as mm


def test_printed_7p5b_nd64(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "memory_model_7p5b_nd64.json")))
    for stage, gb in d["printed_gb"].items():
        got = mm.bytes_per_device(d["psi"], d["nd"], int(stage))
        assert round(got / 1e9, 1) == gb, (stage, got)


def test_exact_7p5b_nd64():
    psi = 7.5e9
    assert mm.bytes_per_device(psi, 64, 0) == 120e9
    assert mm.bytes_per_device(psi, 64, 1) == 31.40625e9
    assert mm.bytes_per_device(psi, 64, 2) == 16.640625e9
    assert mm.bytes_per_device(psi, 64, 3) == 1.875e9


def test_sixteen_bytes_per_param():
    # 2 (fp16 params) + 2 (fp16 grads) + 12 (fp32 master, m, v)
    for psi in (1, 1 << 20, 1.4e9, 13e9, 1e11):
        assert mm.bytes_per_device(psi, 64, 0) == 16 * psi
        assert mm.bytes_per_device(psi, 1, 3) == 16 * psi
    assert mm.bytes_per_device(1 << 20, 4, 0) == 16_777_216
    assert mm.bytes_per_device(1.4e9, 1, 0) == 22.4e9


def test_nd1_every_stage_is_plain_dp():
    for stage in range(4):
        assert mm.bytes_per_device(1e9, 1, stage) == 16e9


def test_reduction_limits():
    psi = 1e9
    big = 10 ** 12
    dp = mm.bytes_per_device(psi, big, 0)
    assert abs(dp / mm.bytes_per_device(psi, big, 1) - 4.0) < 1e-9
    assert abs(dp / mm.bytes_per_device(psi, big, 2) - 8.0) < 1e-9
    # never beyond the limits at any finite Nd
    for nd in (2, 8, 64, 400, 4096):
        assert dp / mm.bytes_per_device(psi, nd, 1) < 4.0
        assert dp / mm.bytes_per_device(psi, nd, 2) < 8.0


def test_stage3_linear_in_nd():
    psi = 7.5e9
    for nd in (1, 2, 3, 64, 400):
        assert mm.bytes_per_device(psi, nd, 3) * nd == pytest.approx(16 * psi, rel=1e-15)


def test_stages_monotone():
    for nd in (2, 4, 64):
        b = [mm.bytes_per_device(7.5e9, nd, s) for s in range(4)]
        assert b[0] > b[1] > b[2] > b[3]


def test_13b_nd32_stage2():
    # 13B at Nd = 32 in stage 2: 2 Psi + 14 Psi / 32
    assert mm.bytes_per_device(13e9, 32, 2) == 31.6875e9


@pytest.mark.parametrize("nd,stage", [(0, 0), (4, -1), (4, 4)])
def test_bad_args(nd, stage):
    with pytest.raises(ValueError):
        mm.bytes_per_device(1e9, nd, stage)
