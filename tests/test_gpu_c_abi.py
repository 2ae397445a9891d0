"""The boundary from plain C: tests/native/abi_gpu_driver.c (built by
tests/native/build_driver.py) reduces one bucket and runs Adam steps through
include/zero.h alone, on hipMalloc'd memory and a HIP stream of its own, in a
process with no Python or torch.  Its outputs must equal the oracle bit for bit:
the reduced gradient (zeros outside the bucket), master, m and v after the
steps, and the whole fp16 vector (the rank's slot, zeros elsewhere).  The rows'
stride padding holds NaN patterns, so a read outside the bucket would show."""
import os
import struct
import subprocess

import numpy as np
import pytest

import zero_sharded_mixed_bucketed_amd as Z
from conftest import ROOT
from gpu_util import assert_bits, need_gpu
from oracle import adam as oadam
from oracle import reduce as ored
from synth import gen

pytestmark = pytest.mark.gpu
EXE = os.path.join(ROOT, "tests", "native", "build", "abi_gpu_driver")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


@pytest.mark.parametrize("psi,nd,rank,boff,blen", [(100_003, 5, 2, 30_000, 25_000),
                                                   (65_536, 4, 3, 0, 65_536),
                                                   (10_007, 7, 0, 1_000, 999)])
def test_c_consumer_matches_the_oracle(tmp_path, psi, nd, rank, boff, blen):
    assert os.path.exists(EXE), "tests/native/build/abi_gpu_driver is not built; run build()"
    seed, steps, lr, b1, b2, eps = 77 + rank, 3, 1e-3, 0.9, 0.999, 1e-8
    geom = Z.shard_geometry(psi, nd, rank)
    lo, S = geom.offset, geom.len
    stride = Z.row_stride(blen)
    rows = gen.grad_rows(seed, nd, boff, boff + blen, 1e-3)
    padded = np.full((nd, stride), 0x7E01, dtype=np.uint16)     # NaN in the padding
    padded[:, :blen] = rows
    flat = np.arange(lo, lo + S, dtype=np.uint64)
    th = gen.state_f32(seed, gen.KIND_MASTER, flat, 0.02)
    m = gen.state_f32(seed, gen.KIND_M, flat, 1e-4)
    v = gen.state_f32(seed, gen.KIND_V, flat, 1e-6, True)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<QIIQQQII4d", psi, nd, rank, boff, blen, stride, steps, 0,
                            lr, b1, b2, eps))
        f.write(padded.tobytes())
        for a in (th, m, v):
            f.write(a.astype("<f4").tobytes())
    dst = tmp_path / "out.bin"
    print(f"c driver psi={psi} nd={nd} rank={rank} bucket=[{boff}, +{blen})", flush=True)
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi gpu driver ok" in r.stdout
    out = np.fromfile(dst, dtype=np.uint8)
    assert out.size == 16 * S + 2 * psi
    got_g = out[:4 * S].view(np.float32)
    got_th, got_m, got_v = (out[4 * S * k:4 * S * (k + 1)].view(np.float32) for k in (1, 2, 3))
    got_p = out[16 * S:].view(np.uint16)

    want_g = np.zeros(S, np.float32)
    ored.reduce_shard(psi, nd, rank, boff, blen, rows, want_g)
    p16 = None
    for t in range(1, steps + 1):
        th, m, v, p16 = oadam.step_values(th, m, v, want_g, oadam.scalars(lr, b1, b2, eps, t))
    want_p = np.zeros(psi, np.uint16)
    want_p[lo:lo + S] = p16
    assert_bits(got_g, want_g, "reduced gradient")
    assert_bits(got_th, th, "master")
    assert_bits(got_m, m, "m")
    assert_bits(got_v, v, "v")
    assert_bits(got_p, want_p, "fp16 vector")
