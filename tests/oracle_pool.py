"""The oracle over a whole shard, chunk by chunk, in a pool of fresh interpreters.

A full-state comparison at the workloads' real sizes needs the oracle over
every element (117,187,500 at the 7.5B / Nd = 64 rank): the reduce of the Nd
seeded fp16 rows and the whole Adam trajectory t = 1..K.  Every step of the
path is element-wise, so the shard splits into chunks that are computed
independently, in one process per host core ("spawn": the workers start fresh
interpreters and never touch the GPU).  Each worker regenerates its chunk's
inputs with the host generator, runs the oracle, and returns a SHA-256 digest
per array and step instead of the arrays themselves; the caller hashes the
device results chunk by chunk the same way, so equal digests mean equal bits.

Test infrastructure: this module calls the oracle and is never imported by the
product path.
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
ARRAYS = ("master", "m", "v", "p16")


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def workers() -> int:
    """One process per available host core, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def chunk_inputs(w, flat):
    """The seeded inputs at flat indices: the Nd fp16 rows (for plain data
    parallelism, the one raw fp16 gradient) and the initial state."""
    from synth import gen
    if w.fp16_grad:
        rows = gen.grad_f16(w.seed, 0, flat, w.grad.sigma, w.grad.heavy_tail,
                            kind=gen.KIND_GRAD_FULL)[None, :]
    else:
        rows = np.empty((w.nd, flat.size), np.uint16)
        for k in range(w.nd):
            rows[k] = gen.grad_f16(w.seed, k, flat, w.grad.sigma, w.grad.heavy_tail)
    state = (gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma),
             gen.state_f32(w.seed, gen.KIND_M, flat, w.m.sigma, w.m.absolute),
             gen.state_f32(w.seed, gen.KIND_V, flat, w.v.sigma, w.v.absolute))
    return rows, state


def chunk_gradient(w, rows):
    """The gradient Adam reads: the reduced fp32 shard, its fp16 copy for an fp16
    shard, or the raw fp16 gradient of plain data parallelism."""
    from oracle import reduce as ored
    if w.fp16_grad:
        return rows[0]
    g = ored.reduce_values(rows, w.nd)
    return g.astype(np.float16).view(np.uint16) if w.grad_shard == "fp16" else g


def chunk_trajectory(job):
    """In a worker: digests of the gradient Adam reads (key ("grad", 0)) and of
    master, m, v and the fp16 parameters after each step t = 1..steps, for
    shard-local elements [j0, j0 + n)."""
    from oracle import adam as oadam
    w, offset, j0, n, steps = job
    flat = np.arange(offset + j0, offset + j0 + n, dtype=np.uint64)
    rows, (th, m, v) = chunk_inputs(w, flat)
    g = chunk_gradient(w, rows)
    del rows
    out = {("grad", 0): digest(g)}
    for t in range(1, steps + 1):
        th, m, v, p16 = oadam.step_values(th, m, v, g,
                                          oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t))
        for name, a in zip(ARRAYS, (th, m, v, p16)):
            out[(name, t)] = digest(a)
    return j0, out


def chunks(length: int, chunk: int = CHUNK):
    return [(j0, min(chunk, length - j0)) for j0 in range(0, length, chunk)]


class ShardOracle:
    """Starts the oracle's digests of a whole shard in the background; result()
    waits for them: {(array, step): {chunk start: digest}}."""

    def __init__(self, w, offset: int, length: int, steps: int, chunk: int = CHUNK):
        self.chunks = chunks(length, chunk)
        jobs = [(w, offset, j0, n, steps) for j0, n in self.chunks]
        self._pool = mp.get_context("spawn").Pool(workers())
        self._it = self._pool.imap_unordered(chunk_trajectory, jobs, chunksize=1)

    def result(self, timeout: float = 900.0, progress_s: float = 20.0):
        """Waits for every chunk, printing how many are done every `progress_s`
        seconds (a whole shard takes minutes); raises TimeoutError after
        `timeout` seconds."""
        n = len(self.chunks)
        parts = []
        t0 = last = time.monotonic()
        try:
            while len(parts) < n:
                try:
                    parts.append(self._it.next(timeout=1.0))
                except mp.TimeoutError:
                    pass
                now = time.monotonic()
                if now - t0 > timeout:
                    raise TimeoutError(f"oracle pool: {len(parts)} of {n} chunks after "
                                       f"{timeout:.0f} s")
                if now - last >= progress_s:
                    print(f"oracle pool: {len(parts)} of {n} chunks done", flush=True)
                    last = now
        finally:
            self._pool.terminate()
            self._pool.join()
        out = {}
        for j0, d in parts:
            for key, h in d.items():
                out.setdefault(key, {})[j0] = h
        return out

    def close(self):
        self._pool.terminate()
        self._pool.join()


def chunk_digests(a: np.ndarray, spans, threads: int = 16):
    """{chunk start: digest} of a host array over the chunk spans (hashlib
    releases the interpreter lock, so threads hash in parallel)."""
    with ThreadPoolExecutor(threads) as ex:
        hs = list(ex.map(lambda s: digest(a[s[0]:s[0] + s[1]]), spans))
    return {j0: h for (j0, _), h in zip(spans, hs)}
