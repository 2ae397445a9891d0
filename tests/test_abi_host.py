"""The C ABI on the host (no GPU needed): the library loads and exports every
symbol include/zero.h declares; its host functions (memory model, geometry,
scalars) agree with the oracle bit for bit; every argument error is rejected
before any device work.  No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import zero_sharded_mixed_bucketed_amd as Z
from conftest import ROOT
from oracle import adam as oadam
from oracle import comm_model as ocm
from oracle import geometry as ogeo
from oracle import memory_model as omm


def _declared():
    text = open(os.path.join(ROOT, "include", "zero.h")).read()
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", Z.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (zero_[a-z0-9_]+)", out))
    declared = set(_declared())
    assert declared == set(Z.EXPORTS)
    assert declared <= exported, declared - exported
    for name in declared:
        assert hasattr(Z.lib, name)


def test_row_stride_rule():
    """Rows start on 128-byte lines, and no stride is a whole number of MiB (such
    strides get 2 KiB more); otherwise nothing is added."""
    assert Z.row_stride(0) == 0
    assert Z.row_stride(1) == 64
    assert Z.row_stride(64) == 64
    assert Z.row_stride(65) == 128
    assert Z.row_stride(25_000_000) == 25_000_000
    assert Z.row_stride(17_187_500) == 17_187_520
    assert Z.row_stride(1 << 22) == (1 << 22) + 1024           # 8 MiB rows
    assert Z.row_stride((1 << 22) - 5) == (1 << 22) + 1024
    assert Z.row_stride(1 << 19) == (1 << 19) + 1024           # 1 MiB rows
    assert Z.row_stride(3 << 19) == (3 << 19) + 1024           # 3 MiB rows
    assert Z.row_stride((1 << 19) + 1) == (1 << 19) + 64
    rng = np.random.default_rng(5)
    for n in list(rng.integers(1, 1 << 40, size=2000)) + [k << 19 for k in range(1, 300)]:
        n = int(n)
        s = Z.row_stride(n)
        assert s >= n and s % 64 == 0 and (s * 2) % (1 << 20) != 0
        assert s - n < 64 + 1024
        if ((n + 63) // 64 * 64 * 2) % (1 << 20):
            assert s == (n + 63) // 64 * 64
    with pytest.raises(Z.ZeroError):
        Z.row_stride((1 << 64) - 1)
    assert Z.row_stride((1 << 64) - 1088) % 64 == 0


def test_memory_model_matches_oracle_and_print():
    for psi in (1 << 20, 1_400_000_000, 7_500_000_000, 13_000_000_000, 10 ** 11):
        for nd in (1, 4, 32, 64, 400):
            for st in range(4):
                assert Z.memory_model(psi, nd, st) == omm.bytes_per_device(psi, nd, st)
    assert [round(Z.memory_model(7_500_000_000, 64, s) / 1e9, 1) for s in range(4)] == \
        [120.0, 31.4, 16.6, 1.9]


def test_memory_model_k_matches_oracle():
    for psi in (1 << 20, 7_500_000_000, 10 ** 11):
        for nd in (1, 4, 64, 400):
            for st in range(4):
                for k in (0.0, 4.0, 12.0, 16.0, 14.5):
                    assert Z.memory_model_k(psi, nd, st, k) == omm.bytes_per_device(psi, nd, st, k)
                assert Z.memory_model_k(psi, nd, st, 12.0) == Z.memory_model(psi, nd, st)
    for bad in (-1.0, float("nan"), float("inf")):
        with pytest.raises(Z.ZeroError):
            Z.memory_model_k(100, 4, 0, bad)


def test_comm_volume_matches_oracle():
    for psi in (1, 1 << 20, 7_500_000_000, 10 ** 11):
        for nd in (1, 2, 3, 64, 400):
            for st in range(4):
                c = Z.comm_volume(psi, nd, st)
                o = ocm.comm_volume(psi, nd, st)
                assert c.reduce_scatters == o.collectives.count("reduce_scatter")
                assert c.all_gathers == o.collectives.count("all_gather")
                assert c.elems == o.elems
                assert c.elems_sent_per_rank == o.elems_sent_per_rank
                assert c.bytes_sent_per_rank == o.bytes_sent_per_rank
    for nd, st in ((0, 0), (4, -1), (4, 4)):
        with pytest.raises(Z.ZeroError):
            Z.comm_volume(100, nd, st)


def test_memory_model_rejects():
    with pytest.raises(Z.ZeroError):
        Z.memory_model(100, 0, 0)
    with pytest.raises(Z.ZeroError):
        Z.memory_model(100, 4, 4)


@pytest.mark.parametrize("psi", [1, 7, 37, 1000, 1 << 20, 7_500_000_000, 10 ** 11,
                                 2 ** 64 - 1, 2 ** 64 - 3, 2 ** 63 + 5])
@pytest.mark.parametrize("nd", [1, 3, 4, 7, 64, 400])
def test_geometry_matches_oracle(psi, nd):
    ranks = range(nd) if nd <= 64 else (0, 1, 137, nd - 1)
    for r in ranks:
        g = Z.shard_geometry(psi, nd, r)
        lo, hi = ogeo.shard_range(psi, nd, r)
        assert (g.offset, g.len) == (lo, hi - lo)


def test_bucket_intersect():
    g = Z.shard_geometry(100, 4, 1)                 # [25, 50)
    assert Z.bucket_intersect(g, 0, 10) == (25, 25)
    assert Z.bucket_intersect(g, 20, 10) == (25, 30)
    assert Z.bucket_intersect(g, 30, 5) == (30, 35)
    assert Z.bucket_intersect(g, 40, 60) == (40, 50)
    with pytest.raises(Z.ZeroError) as e:
        Z.bucket_intersect(g, 95, 10)
    assert e.value.code == Z.ZERO_E_RANGE


@pytest.mark.parametrize("lr,b1,b2,eps", [(1e-3, 0.9, 0.999, 1e-8), (1e-4, 0.9, 0.999, 1e-8),
                                          (3e-4, 0.8, 0.95, 1e-6), (1.0, 0.0, 0.5, 1e-3)])
@pytest.mark.parametrize("t", [1, 2, 3, 7, 10, 20, 1000, 10 ** 6])
def test_scalars_match_oracle_bits(lr, b1, b2, eps, t):
    got = np.array(Z.adam_scalars(lr, b1, b2, eps, t), dtype=np.float32)
    want = np.array(oadam.scalars(lr, b1, b2, eps, t).as_tuple(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("args", [
    (1e-3, 0.9, 0.999, 1e-8, 0),          # step 0
    (1e-3, 1.0, 0.999, 1e-8, 1),          # beta1 = 1
    (1e-3, 0.9, -0.1, 1e-8, 1),           # beta2 < 0
    (1e-3, 0.9, 0.999, 0.0, 1),           # eps = 0
    (float("nan"), 0.9, 0.999, 1e-8, 1),  # lr NaN
    (1e-3, 0.9, 0.999, float("inf"), 1),
])
def test_scalars_reject(args):
    with pytest.raises(Z.ZeroError) as e:
        Z.adam_scalars(*args)
    assert e.value.code == Z.ZERO_E_INVAL


def _geom(psi=100, nd=4, rank=1, offset=None, length=None):
    g = Z.Geom()
    g.psi, g.nd, g.rank = psi, nd, rank
    ref = Z.shard_geometry(psi, nd, rank) if nd and rank < nd and psi else None
    g.offset = ref.offset if offset is None and ref else (offset or 0)
    g.len = ref.len if length is None and ref else (length or 0)
    return g


FAKE = 0x10000     # never dereferenced: every call below is rejected first


def _reduce(g, off=25, n=25, slices=FAKE, stride=25, g32=FAKE, g16=None):
    return Z.lib.zero_reduce_shard(ctypes.byref(g), off, n, slices, stride, g32, g16, None)


@pytest.mark.parametrize("call,code", [
    (lambda: Z.lib.zero_reduce_shard(None, 0, 1, FAKE, 1, FAKE, None, None), Z.ZERO_E_INVAL),
    (lambda: _reduce(_geom(nd=0, offset=0, length=0)), Z.ZERO_E_INVAL),
    (lambda: _reduce(_geom(rank=4, offset=0, length=25)), Z.ZERO_E_INVAL),
    (lambda: _reduce(_geom(offset=26)), Z.ZERO_E_INVAL),          # geometry mismatch
    (lambda: _reduce(_geom(length=24)), Z.ZERO_E_INVAL),
    (lambda: _reduce(_geom(), off=90, n=20), Z.ZERO_E_RANGE),      # beyond psi
    (lambda: _reduce(_geom(), off=2 ** 64 - 5, n=10), Z.ZERO_E_RANGE),
    (lambda: _reduce(_geom(), slices=None), Z.ZERO_E_INVAL),
    (lambda: _reduce(_geom(), g32=None), Z.ZERO_E_INVAL),         # no output at all
    (lambda: _reduce(_geom(), g32=None, g16=FAKE + 1), Z.ZERO_E_ALIGN),
    (lambda: _reduce(_geom(), stride=24), Z.ZERO_E_RANGE),
    (lambda: _reduce(_geom(), stride=2 ** 63), Z.ZERO_E_RANGE),    # size overflow
    (lambda: _reduce(_geom(), slices=FAKE + 1), Z.ZERO_E_ALIGN),
    (lambda: _reduce(_geom(), g32=FAKE + 2), Z.ZERO_E_ALIGN),
    (lambda: _reduce(_geom(), g16=FAKE + 1), Z.ZERO_E_ALIGN),
    # Nd above 2^24, where fp32(Nd) is no longer Nd, for a bucket that meets the shard
    (lambda: _reduce(_geom(psi=1 << 30, nd=(1 << 24) + 1, rank=0), off=0, n=10),
     Z.ZERO_E_RANGE),
])
def test_reduce_rejects(call, code):
    assert call() == code
    assert Z.last_error()


def test_reduce_empty_intersection_is_ok_without_device():
    # bucket [0, 10) does not meet shard [25, 50): no device call at all
    assert _reduce(_geom(), off=0, n=10, slices=None, g32=None) == Z.ZERO_OK
    assert _reduce(_geom(), off=25, n=0) == Z.ZERO_OK


def _shard(grad16=0, p16=FAKE, origin=0, plen=100, master=FAKE, grad=FAKE):
    s = Z.Shard()
    s.master, s.m, s.v, s.grad = master, FAKE, FAKE, grad
    s.grad_is_fp16 = grad16
    s.param16, s.param16_origin, s.param16_len = p16, origin, plen
    return s


def _adam(g, s, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, t=1):
    return Z.lib.zero_adam_step_shard(ctypes.byref(g), ctypes.byref(s) if s else None, lr, b1,
                                      b2, eps, t, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _adam(_geom(offset=3), _shard()), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), None), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(), t=0), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(), b1=1.5), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(), eps=-1.0), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(master=None)), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(grad=None)), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(grad16=2)), Z.ZERO_E_INVAL),
    (lambda: _adam(_geom(), _shard(origin=30, plen=70)), Z.ZERO_E_RANGE),   # slot starts before window
    (lambda: _adam(_geom(), _shard(origin=0, plen=49)), Z.ZERO_E_RANGE),    # slot ends after it
    (lambda: _adam(_geom(), _shard(origin=26, plen=10 ** 6)), Z.ZERO_E_RANGE),
    (lambda: _adam(_geom(), _shard(master=FAKE + 2)), Z.ZERO_E_ALIGN),
    (lambda: _adam(_geom(), _shard(grad=FAKE + 2)), Z.ZERO_E_ALIGN),
    (lambda: _adam(_geom(), _shard(grad16=1, grad=FAKE + 1)), Z.ZERO_E_ALIGN),
    (lambda: _adam(_geom(), _shard(p16=FAKE + 1)), Z.ZERO_E_ALIGN),
])
def test_adam_rejects(call, code):
    assert call() == code
    assert Z.last_error()


def test_adam_empty_trailing_shard_is_ok_without_device():
    g = Z.shard_geometry(10, 16, 15)        # S = 1: ranks 10..15 own nothing
    assert g.len == 0
    assert _adam(g, _shard(master=None, grad=None)) == Z.ZERO_OK


def test_one_hip_runtime_in_process():
    # libzero and the synthetic-input library resolve to torch's HIP runtime
    from synth import device as sdev
    sdev._load()
    assert len(Z.hip_runtimes()) == 1, Z.hip_runtimes()


def _gather(psi=100, nd=4, lo=10, n=20, shards=FAKE, stride=25, out=FAKE):
    return Z.lib.zero_gather_params(psi, nd, lo, n, shards, stride, out, None)


@pytest.mark.parametrize("call,code", [
    (lambda: _gather(nd=0), Z.ZERO_E_INVAL),
    (lambda: _gather(psi=0), Z.ZERO_E_INVAL),
    (lambda: _gather(lo=90, n=11), Z.ZERO_E_RANGE),                # beyond psi
    (lambda: _gather(lo=2 ** 64 - 5, n=10), Z.ZERO_E_RANGE),
    (lambda: _gather(shards=None), Z.ZERO_E_INVAL),
    (lambda: _gather(out=None), Z.ZERO_E_INVAL),
    (lambda: _gather(stride=24), Z.ZERO_E_RANGE),                  # stride < S = 25
    (lambda: _gather(stride=2 ** 63), Z.ZERO_E_RANGE),             # size overflow
    (lambda: _gather(shards=FAKE + 1), Z.ZERO_E_ALIGN),
    (lambda: _gather(out=FAKE + 1), Z.ZERO_E_ALIGN),
])
def test_gather_rejects(call, code):
    assert call() == code
    assert Z.last_error()


def test_gather_empty_is_ok_without_device():
    assert _gather(n=0, shards=None, out=None) == Z.ZERO_OK
    assert _gather(lo=100, n=0) == Z.ZERO_OK


def test_c_consumer_links_and_rejects_bad_input(tmp_path):
    """The plain C consumer of the library starts (its libzero.so and HIP runtime
    resolve) and refuses a bad command line or a short input before any device
    call."""
    exe = os.path.join(ROOT, "tests", "native", "build", "abi_gpu_driver")
    assert os.path.exists(exe), "not built; run __graft_entry__.build()"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=30)
    assert r.returncode == 2 and "usage" in r.stderr
    short = tmp_path / "short.bin"
    short.write_bytes(b"\x00" * 10)
    r = subprocess.run([exe, str(short), str(tmp_path / "out.bin")], capture_output=True,
                       text=True, timeout=30)
    assert r.returncode == 2 and "short input" in r.stderr


def test_binding_requires_one_device_per_call():
    """Every tensor of a call and its stream must share one device (checked on
    stand-ins; the library launches on that device)."""
    from types import SimpleNamespace as NS
    import torch
    a, b = torch.device("cuda", 0), torch.device("cuda", 1)
    assert Z._one_device([NS(device=a), NS(device=a)], None) == a
    assert Z._one_device([NS(device=a)], NS(device=a)) == a
    with pytest.raises(ValueError):
        Z._one_device([NS(device=a), NS(device=b)], None)
    with pytest.raises(ValueError):
        Z._one_device([NS(device=a)], NS(device=b))


def test_last_error_is_per_thread():
    """Concurrent failing calls (ctypes drops the GIL around them): each thread
    reads back the message of its own last error."""
    import threading
    errors = []

    def worker(i):
        g = _geom()
        for _ in range(2000):
            # stride 24 + i < bucket length 25 + i: the message names both values
            rc = Z.lib.zero_reduce_shard(ctypes.byref(g), 25, 25, FAKE, 24 - (i % 20), FAKE,
                                         None, None)
            msg = Z.last_error()
            if rc != Z.ZERO_E_RANGE or f"slice_stride {24 - (i % 20)} " not in msg:
                errors.append((i, rc, msg))
                return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_launch_occupancy_rejects_before_any_device_call():
    """An unknown kernel or a NULL output is refused before the library asks for
    the device (no GPU here)."""
    wgs, lds = ctypes.c_int(-7), ctypes.c_uint32(7)
    for kernel in (-1, 6, 1000):
        assert Z.lib.zero_launch_occupancy(kernel, ctypes.byref(wgs), ctypes.byref(lds)) \
            == Z.ZERO_E_INVAL
        assert "unknown kernel" in Z.last_error()
    assert Z.lib.zero_launch_occupancy(Z.KERNEL_REDUCE_W16, None, ctypes.byref(lds)) \
        == Z.ZERO_E_INVAL
    assert (wgs.value, lds.value) == (-7, 7)
