"""Planted mistakes in the oracle (on the CPU) must fail at least one pin.

Each mutant below is a plausible slip -- a dropped term, a wrong sign, swapped
operands, another order or rounding -- patched into the oracle for the span
of one test; the pin tests are then run against it and must raise.
"""
import math

import numpy as np
import pytest

import test_oracle_adam as pins_adam
import test_oracle_reduce as pins_reduce
from oracle import adam, reduce as red


def _step(mutation):
    def step_values(master, m, v, grad, sc):
        g = adam.grad_f32(grad)
        b1, b2, c1, c2, eps, step, isb = sc.as_tuple()
        if mutation == "swap_betas":
            b1, b2, c1, c2 = b2, b1, c2, c1
        m_new = b1 * m + c1 * g
        if mutation == "g_not_squared":
            v_new = b2 * v + c2 * np.abs(g)
        else:
            v_new = b2 * v + c2 * (g * g)
        if mutation == "eps_inside_sqrt":
            den = np.sqrt(v_new * isb * isb + eps)
        elif mutation == "no_v_bias_correction":
            den = np.sqrt(v_new) + eps
        else:
            den = np.sqrt(v_new) * isb + eps
        upd = step * (m_new / den)
        if mutation == "old_moment":
            upd = step * (m / den)
        th = master + upd if mutation == "wrong_sign" else master - upd
        return th, m_new, v_new, th.astype(np.float16).view(np.uint16)
    return step_values


ADAM_MUTANTS = ["swap_betas", "g_not_squared", "eps_inside_sqrt", "no_v_bias_correction",
                "old_moment", "wrong_sign"]


@pytest.mark.parametrize("mutation", ADAM_MUTANTS)
def test_adam_mutants_fail_the_textbook_shadow(monkeypatch, mutation):
    monkeypatch.setattr(adam, "step_values", _step(mutation))
    with pytest.raises(AssertionError):
        for case in [(1e-4, 1e-6, 1e-3, 1e-4, False), (0.0, 0.0, 5e-3, 1e-3, False)]:
            pins_adam.test_against_fp64_textbook(case)


def _scalars(mutation):
    real = adam.scalars

    def scalars(lr, beta1, beta2, eps, t):
        sc = real(lr, beta1, beta2, eps, t)
        if mutation == "no_m_bias_correction":
            return adam.Scalars(sc.b1, sc.b2, sc.c1, sc.c2, sc.eps, np.float32(lr), sc.isb)
        if mutation == "one_minus_beta_in_fp32":
            c1 = np.float32(1.0) - np.float32(beta1)
            c2 = np.float32(1.0) - np.float32(beta2)
            return adam.Scalars(sc.b1, sc.b2, c1, c2, sc.eps, sc.step, sc.isb)
        if mutation == "t_from_zero":
            return real(lr, beta1, beta2, eps, t + 1)
        if mutation == "sqrt_not_inverted":
            return adam.Scalars(sc.b1, sc.b2, sc.c1, sc.c2, sc.eps, sc.step,
                                np.float32(math.sqrt(1.0 - beta2 ** t)))
        raise AssertionError(mutation)
    return scalars


@pytest.mark.parametrize("mutation", ["no_m_bias_correction", "one_minus_beta_in_fp32",
                                      "t_from_zero", "sqrt_not_inverted"])
def test_scalar_mutants_fail_a_pin(monkeypatch, mutation):
    monkeypatch.setattr(adam, "scalars", _scalars(mutation))
    failed = 0
    for fn in (lambda: pins_adam.test_scalars_against_exact(1e-3, 0.9, 0.999, 1e-8, 1),
               lambda: pins_adam.test_against_fp64_textbook((1e-4, 1e-6, 1e-3, 1e-4, False)),
               pins_adam.test_closed_form_constant_gradient):
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed >= 1


def _reduce(mutation):
    def reduce_values(rows, nd):
        rows = np.asarray(rows)
        x = [rows[k].view(np.float16).astype(np.float32) for k in range(nd)]
        if mutation == "descending_order":
            x = x[::-1]
        if mutation == "start_from_first":
            acc = x[0].copy()
            rest = x[1:]
        else:
            acc = np.zeros(rows.shape[1], np.float32)
            rest = x
        for xk in rest:
            acc = acc + xk
        if mutation == "divide":
            return acc / np.float32(nd)
        if mutation == "no_scale":
            return acc
        if mutation == "pairwise":
            return np.sum(np.stack(x), axis=0, dtype=np.float32) * red.inv_nd(nd)
        return acc * red.inv_nd(nd)
    return reduce_values


@pytest.mark.parametrize("mutation", ["descending_order", "start_from_first", "divide",
                                      "no_scale"])
def test_reduce_mutants_fail_a_pin(monkeypatch, mutation, golden_dir):
    monkeypatch.setattr(red, "reduce_values", _reduce(mutation))
    failed = 0
    for fn in (lambda: pins_reduce.test_hand_worked_cases(golden_dir),
               lambda: pins_reduce.test_closed_form(3, 0.01),
               lambda: pins_reduce.test_closed_form(4, 0.01)):
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_reduce_shard_offset_mutant_fails(monkeypatch):
    real = red.reduce_shard

    def shifted(psi, nd, rank, off, n, rows, g32, g16=None):
        return real(psi, nd, rank, off, n, np.roll(rows, 1, axis=1), g32, g16)
    monkeypatch.setattr(red, "reduce_shard", shifted)
    with pytest.raises(AssertionError):
        pins_reduce.test_brute_force_all_ranks(37, 3, 10)


# ---- communication and K-general memory model ---------------------------------------

import test_oracle_comm_model as pins_comm  # noqa: E402
from oracle import comm_model as cm  # noqa: E402
from oracle import memory_model as mm  # noqa: E402


def _comm(mutation):
    real = cm.comm_volume

    def comm_volume(psi, nd, stage):
        c = real(psi, nd, stage)
        if mutation == "stage3_one_all_gather" and stage == 3:
            return cm.Comm(("all_gather", "reduce_scatter"), 2 * psi, 2 * psi * (nd - 1) / nd)
        if mutation == "no_ring_factor":
            return cm.Comm(c.collectives, c.elems, c.elems)
        if mutation == "stage1_all_reduce_plus_gather" and stage == 1:
            return cm.Comm(("reduce_scatter", "all_gather", "all_gather"), 3 * psi,
                           3 * psi * (nd - 1) / nd)
        return c
    return comm_volume


@pytest.mark.parametrize("mutation", ["stage3_one_all_gather", "no_ring_factor",
                                      "stage1_all_reduce_plus_gather"])
def test_comm_mutants_fail_a_pin(monkeypatch, mutation):
    monkeypatch.setattr(cm, "comm_volume", _comm(mutation))
    failed = 0
    checks = [pins_comm.test_pages_counts, pins_comm.test_exact_limits,
              lambda: [pins_comm.test_exact_per_rank_volume_by_ring_count(nd, st)
                       for nd in (2, 3) for st in range(4)]]
    for fn in checks:
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed, mutation


def _mem(mutation):
    real = mm.bytes_per_device

    def bytes_per_device(psi, nd, stage, k=mm.K_ADAM):
        if mutation == "k_on_grads_too" and stage == 2:
            return 2 * psi + (2 * k + k) * psi / nd / 2 + 0.5 * k * psi / nd
        if mutation == "stage1_grads_sharded" and stage == 1:
            return 2 * psi + (2 + k) * psi / nd
        if mutation == "fixed_k" and k != mm.K_ADAM:
            return real(psi, nd, stage, mm.K_ADAM)
        return real(psi, nd, stage, k)
    return bytes_per_device


@pytest.mark.parametrize("mutation", ["k_on_grads_too", "stage1_grads_sharded", "fixed_k"])
def test_memory_k_mutants_fail_a_pin(monkeypatch, mutation):
    monkeypatch.setattr(mm, "bytes_per_device", _mem(mutation))
    failed = 0
    for fn in (lambda: [pins_comm.test_memory_k_brute_force(k, nd, st)
                        for k in (4, 12) for nd in (2, 4) for st in range(4)],
               lambda: [pins_comm.test_memory_k_limits(k) for k in (4, 12, 20)]):
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed, mutation


# ---- stage-3 parameter gather ---------------------------------------------------------

import test_oracle_stage3 as pins_stage3  # noqa: E402
from oracle import geometry as ogeo  # noqa: E402
from oracle import stage3 as st3  # noqa: E402


def _gather(mutation):
    def gather_params(shards, psi, nd, lo, n):
        s = ogeo.shard_size(psi, nd)
        if mutation == "floor_shard_size":
            s = max(1, psi // nd)
        i = np.arange(lo, lo + n, dtype=np.int64)
        k = i // s
        if mutation == "next_rank":
            k = np.minimum(k + (i % 7 == 3), nd - 1)
        k = np.minimum(k, nd - 1)
        col = i - k * s
        if mutation == "column_from_range_start":
            col = col - (lo % s) * (i == lo)
        return shards[k, np.clip(col, 0, shards.shape[1] - 1)]
    return gather_params


@pytest.mark.parametrize("mutation", ["floor_shard_size", "next_rank", "column_from_range_start"])
def test_gather_mutants_fail_a_pin(monkeypatch, mutation):
    monkeypatch.setattr(st3, "gather_params", _gather(mutation))
    failed = 0
    checks = [lambda: [pins_stage3.test_all_layers_rebuild_the_vector(psi, nd)
                       for psi, nd in ((10, 3), (37, 4), (100, 7), (1000, 64))],
              lambda: [pins_stage3.test_brute_force_owner_scan(psi, nd)
                       for psi, nd in ((10, 3), (37, 4))]]
    for fn in checks:
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed, mutation
