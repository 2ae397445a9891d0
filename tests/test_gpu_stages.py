"""Stages 1 and 2 of one rank on the device, through the C ABI, against the
oracle, with the pages' fp16 gradient accounting (upskillscore guide "ZeRO:
particionar estados do treino entre GPUs", section "Como funciona": stage 1
keeps the full gradient, 4 Psi + 12 Psi / Nd; stage 2 only the owned gradient
partition, 2 Psi + 14 Psi / Nd).

* stage 2 with an fp16 gradient shard: the reduce writes only fp16 and Adam
  reads it (28 B/element);
* stage 1: the reduced slice overwrites the rank's own retained local gradient
  in place (its output aliases row `rank` column for column);
* both equal the oracle bit for bit and each other;
* the device memory a step peaks at is the model's resident bytes plus what
  the simulation holds for the other ranks (stage 1: their full local
  gradients; stage 2: one bucket of rows at a time, released after its reduce).
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_bits, f32, need_gpu, rows_device, u16
from oracle import adam as oadam
from oracle import reduce as ored
from synth import device as sdev
from synth import gen, workloads as wl
from zero_sharded_mixed_bucketed_amd import rank as zr

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


def _init_state(st, seed):
    lo = st.geom.offset
    sdev.fill_state(st.master, seed, gen.KIND_MASTER, lo, 0.02)
    sdev.fill_state(st.m, seed, gen.KIND_M, lo, 1e-4)
    sdev.fill_state(st.v, seed, gen.KIND_V, lo, 1e-6, True)


def _oracle(psi, nd, rank, buckets, seed, steps):
    """fp16 gradient shard, then `steps` Adam steps from the same initial state."""
    lo, n = rank * (psi // nd), psi // nd
    w32 = np.zeros(n, np.float32)
    w16 = np.zeros(n, np.uint16)
    for off, blen in buckets:
        rows = gen.grad_rows(seed, nd, off, off + blen, 1e-3)
        ored.reduce_shard(psi, nd, rank, off, blen, rows, w32, w16)
    idx = np.arange(lo, lo + n, dtype=np.uint64)
    th = gen.state_f32(seed, gen.KIND_MASTER, idx, 0.02)
    m = gen.state_f32(seed, gen.KIND_M, idx, 1e-4)
    v = gen.state_f32(seed, gen.KIND_V, idx, 1e-6, True)
    for t in range(1, steps + 1):
        th, m, v, p16 = oadam.step_values(th, m, v, w16, oadam.scalars(LR, B1, B2, EPS, t))
    return w16, th, m, v, p16


@pytest.mark.parametrize("psi,nd,rank,bucket", [(600_012, 4, 1, 100_003),
                                                (600_012, 4, 3, 77_777),
                                                (1 << 20, 8, 5, 1 << 16)])
def test_stage1_in_place_and_stage2_fp16_shard_match_the_oracle(psi, nd, rank, bucket):
    print(f"stages psi={psi} nd={nd} rank={rank} bucket={bucket}", flush=True)
    seed, steps = 515 + rank, 3
    buckets = wl.uniform_buckets(psi, bucket)
    everyone = rows_device(seed, nd, 0, psi, wl.Dist(1e-3))    # [nd][psi]: all local grads
    s2 = zr.RankState(psi, nd, rank, 2)
    s1 = zr.RankState(psi, nd, rank, 1, local_grad=everyone[rank])
    for st in (s2, s1):
        _init_state(st, seed)
    touching = wl.buckets_touching(buckets, s2.geom.offset, s2.geom.offset + s2.geom.len)
    for off, n in touching:                       # stage 2 first: it only reads the rows
        s2.reduce_bucket(off, n, everyone[:, off:off + n])
    for off, n in touching:                       # stage 1 overwrites row `rank` in place
        s1.reduce_bucket(off, n, everyone[:, off:off + n])
    for t in range(1, steps + 1):
        s2.adam_step(LR, B1, B2, EPS, t)
        s1.adam_step(LR, B1, B2, EPS, t)
    torch.cuda.synchronize()
    w16, th, m, v, p16 = _oracle(psi, nd, rank, touching, seed, steps)
    lo, n = s2.geom.offset, s2.geom.len
    for st, name in ((s2, "stage 2"), (s1, "stage 1")):
        assert_bits(u16(st.grad), w16, f"{name} fp16 gradient shard")
        assert_bits(f32(st.master), th, f"{name} master")
        assert_bits(f32(st.m), m, f"{name} m")
        assert_bits(f32(st.v), v, f"{name} v")
        assert_bits(u16(st.param16)[lo:lo + n], p16, f"{name} fp16 slot")
    # stage 1 touched only its own slice of its local gradient
    before = gen.grad_rows(seed, nd, 0, psi, 1e-3)
    after = u16(everyone)
    keep = np.ones(psi, bool)
    keep[lo:lo + n] = False
    assert_bits(after[rank][keep], before[rank][keep], "rest of the own local gradient")
    others = [k for k in range(nd) if k != rank]
    assert_bits(after[others], before[others], "other ranks' local gradients")


def _peak_of(run):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    keep = run()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del keep
    return peak


def test_peak_memory_stage2_is_model_plus_one_bucket():
    psi, nd, rank, bucket = 1 << 20, 4, 2, 1 << 16     # every size a multiple of 512 bytes
    rows_device(1, nd, 0, 256, wl.Dist(1e-3))           # generator tables allocated before
    buckets = wl.uniform_buckets(psi, bucket)

    def run():
        st = zr.RankState(psi, nd, rank, 2)
        lo, n = st.geom.offset, st.geom.len
        for off, blen in wl.buckets_touching(buckets, lo, lo + n):
            rows = rows_device(3, nd, off, blen, wl.Dist(1e-3))     # this bucket arrives
            st.reduce_bucket(off, blen, rows)
            del rows                                                # ... and is released
        st.adam_step(LR, B1, B2, EPS, 1)
        return st
    st_bytes = zr.RankState(psi, nd, rank, 2, device=torch.device("cpu")).resident_bytes()
    assert st_bytes == 2 * psi + 14 * psi // nd
    peak = _peak_of(run)
    assert peak == st_bytes + nd * bucket * 2


def test_peak_memory_stage1_is_model_plus_remote_gradients():
    psi, nd, rank, bucket = 1 << 20, 4, 2, 1 << 16
    rows_device(1, nd, 0, 256, wl.Dist(1e-3))
    buckets = wl.uniform_buckets(psi, bucket)

    def run():
        everyone = rows_device(3, nd, 0, psi, wl.Dist(1e-3))
        st = zr.RankState(psi, nd, rank, 1, local_grad=everyone[rank])
        lo, n = st.geom.offset, st.geom.len
        for off, blen in wl.buckets_touching(buckets, lo, lo + n):
            st.reduce_bucket(off, blen, everyone[:, off:off + blen])
        st.adam_step(LR, B1, B2, EPS, 1)
        return st, everyone
    model = 4 * psi + 12 * psi // nd
    assert zr.RankState(psi, nd, rank, 1, device=torch.device("cpu")).resident_bytes() == model
    peak = _peak_of(run)
    assert peak == model + (nd - 1) * 2 * psi           # the other ranks' local gradients
