"""The chunked oracle pool behind the full-state GPU comparison: on a tiny
workload its per-chunk digests equal the digests of one direct oracle run over
the whole shard, cut into the same chunks (chunking is bit-neutral because
every step is element-wise), and a planted one-bit change is caught."""
import numpy as np

import oracle_pool
from oracle import adam as oadam
from oracle import reduce as ored
from synth import gen
from synth import workloads as wl


def test_pool_digests_equal_a_direct_oracle_run():
    w = wl.tiny()
    lo, S = 0, w.psi // w.nd
    chunk = 1 << 16                                          # 4 chunks
    orc = oracle_pool.ShardOracle(w, lo, S, w.steps, chunk=chunk)
    want = orc.result(timeout=600)
    spans = oracle_pool.chunks(S, chunk)
    assert len(spans) == 4 and sorted(want[("grad", 0)]) == [j0 for j0, _ in spans]
    flat = np.arange(lo, lo + S, dtype=np.uint64)
    g = ored.reduce_values(gen.grad_rows(w.seed, w.nd, lo, lo + S, w.grad.sigma), w.nd)
    assert oracle_pool.chunk_digests(g, spans) == want[("grad", 0)]
    th = gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma)
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    for t in range(1, w.steps + 1):
        th, m, v, p16 = oadam.step_values(th, m, v, g,
                                          oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t))
        for name, a in zip(oracle_pool.ARRAYS, (th, m, v, p16)):
            assert oracle_pool.chunk_digests(a, spans) == want[(name, t)], (name, t)
    # one flipped bit in one chunk changes that chunk's digest only
    th2 = th.copy()
    th2.view(np.uint32)[3 * chunk + 5] ^= 1
    d2 = oracle_pool.chunk_digests(th2, spans)
    assert [j0 for j0, _ in spans if d2[j0] != want[("master", w.steps)][j0]] == [3 * chunk]


def test_pool_fp16_gradients():
    """The raw fp16 gradient of plain data parallelism and an fp16 gradient shard
    are what the pool's chunks digest."""
    from dataclasses import replace
    base = wl.tiny()
    flat = np.arange(0, 1 << 12, dtype=np.uint64)
    plain = replace(base, nd=1, fp16_grad=True, steps=1)
    rows, _ = oracle_pool.chunk_inputs(plain, flat)
    g = oracle_pool.chunk_gradient(plain, rows)
    assert g.dtype == np.uint16 and np.array_equal(
        g, gen.grad_f16(plain.seed, 0, flat, plain.grad.sigma, kind=gen.KIND_GRAD_FULL))
    half = replace(base, grad_shard="fp16")
    rows, _ = oracle_pool.chunk_inputs(half, flat)
    g16 = oracle_pool.chunk_gradient(half, rows)
    assert np.array_equal(g16, ored.reduce_values(rows, half.nd).astype(np.float16)
                          .view(np.uint16))
