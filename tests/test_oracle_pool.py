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
    assert len(spans) == 4 and sorted(want[("grad32", 0)]) == [j0 for j0, _ in spans]
    flat = np.arange(lo, lo + S, dtype=np.uint64)
    g = ored.reduce_values(gen.grad_rows(w.seed, w.nd, lo, lo + S, w.grad.sigma), w.nd)
    assert oracle_pool.chunk_digests(g, spans) == want[("grad32", 0)]
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
