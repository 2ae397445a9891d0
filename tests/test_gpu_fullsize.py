"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times (the same library calls on the same shard sizes), against the oracle on
sampled outputs: every shard edge and bucket edge, plus random picks.  The
oracle regenerates the sampled inputs from the shared generator and computes
them one by one.

Each Adam step is compared from the same input state (the device state at the
samples before the step), so the per-step bar of tests/gpu_util.py applies.
"""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_bucketed_amd as Z
import oracle_pool
from gpu_util import assert_adam_step, assert_bits, gather, need_gpu, sample_indices
from oracle import adam as oadam
from oracle import reduce as ored
from synth import device as sdev
from synth import gen
from synth import workloads as wl

pytestmark = pytest.mark.gpu
N_RANDOM = 1 << 15


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _state(w, geom):
    lo, n = geom.offset, geom.len
    out = []
    for kind, d in ((gen.KIND_MASTER, w.master), (gen.KIND_M, w.m), (gen.KIND_V, w.v)):
        t = torch.empty(n, dtype=torch.float32, device="cuda")
        sdev.fill_state(t, w.seed, kind, lo, d.sigma, d.absolute)
        out.append(t)
    return out


def _host_state(w, flat):
    return (gen.state_f32(w.seed, gen.KIND_MASTER, flat, w.master.sigma),
            gen.state_f32(w.seed, gen.KIND_M, flat, w.m.sigma, w.m.absolute),
            gen.state_f32(w.seed, gen.KIND_V, flat, w.v.sigma, w.v.absolute))


def _reduce_all(w, geom, grad32, chunk=None, grad16=None):
    """Every bucket that meets the shard, in arrival order; only the owned columns
    arrive (rows at the library's advised stride); the rows are freed after each call.
    Returns the shard-local edges of every bucket and of every chunk launch (each
    chunk is a row buffer of its own and starts a new output alignment class)."""
    edges = []
    for off, n in wl.buckets_touching(w.buckets, geom.offset, geom.offset + geom.len):
        a, b = Z.bucket_intersect(geom, off, n)
        edges += [a - geom.offset, b - geom.offset]
        step = chunk or (b - a)
        for c0 in range(a, b, step):
            c1 = min(b, c0 + step)
            edges.append(c0 - geom.offset)
            stride = Z.row_stride(c1 - c0)
            buf = torch.empty(w.nd * stride, dtype=torch.int16, device="cuda")
            rows = buf.as_strided((w.nd, c1 - c0), (stride, 1))
            sdev.fill_grad_rows(rows, w.seed, c0, w.grad.sigma, w.grad.heavy_tail)
            Z.reduce_shard(geom, c0, c1 - c0, rows, grad32, grad16)
            del rows, buf                                # release
    return edges


def _oracle_grad(w, flat):
    rows = np.stack([gen.grad_f16(w.seed, k, flat, w.grad.sigma, w.grad.heavy_tail)
                     for k in range(w.nd)])
    return ored.reduce_values(rows, w.nd)


def _steps(w, geom, state, grad_dev, g_ref, p16, p16_origin, idx, steps, what):
    """Run the Adam steps; compare every step at the samples from the same state."""
    it = torch.from_numpy(idx).cuda()
    pflat = torch.from_numpy(idx + (geom.offset - p16_origin)).cuda()
    master, m, v = state
    for t in range(1, steps + 1):
        before = [x.index_select(0, it).cpu().numpy() for x in state]
        Z.adam_step_shard(geom, master, m, v, grad_dev, p16, p16_origin, w.lr, w.beta1,
                          w.beta2, w.eps, t)
        torch.cuda.synchronize()
        after = [x.index_select(0, it).cpu().numpy() for x in state]
        got_p = p16.index_select(0, pflat).cpu().view(torch.int16).numpy().view(np.uint16)
        sc = oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t)
        want = oadam.step_values(*before, g_ref, sc)
        g32 = oadam.grad_f32(g_ref)
        assert_adam_step((*before, g32), (*after, got_p), want, c1=float(sc.c1),
                         b1=float(sc.b1), b2=float(sc.b2), c2=float(sc.c2),
                         what=f"{what} step {t}")


def _run_zero2(w, chunk=None, window=None):
    geom = Z.shard_geometry(w.psi, w.nd, w.rank)
    print(f"{w.name}: shard [{geom.offset}, +{geom.len})", flush=True)
    state = _state(w, geom)
    grad32 = torch.zeros(geom.len, dtype=torch.float32, device="cuda")
    edges = _reduce_all(w, geom, grad32, chunk)
    torch.cuda.synchronize()
    idx = sample_indices(geom.len, edges, N_RANDOM, seed=w.rank + 17)
    flat = idx.astype(np.uint64) + np.uint64(geom.offset)
    g_ref = _oracle_grad(w, flat)
    assert_bits(gather(grad32, idx).cpu().numpy(), g_ref, f"{w.name} reduced gradient")
    if window is None:
        origin, plen = 0, w.psi
    else:
        origin, plen = geom.offset - window, geom.len + 2 * window
    p16 = torch.zeros(plen, dtype=torch.int16, device="cuda")
    _steps(w, geom, state, grad32, g_ref, p16, origin, idx, w.steps, w.name)
    # nothing written outside the slot: the neighbours of both slot edges are untouched
    lo, hi = geom.offset - origin, geom.offset - origin + geom.len
    for a, b in ((max(0, lo - 4096), lo), (hi, min(plen, hi + 4096))):
        if b > a:
            assert torch.count_nonzero(p16[a:b]).item() == 0
    return geom, state, grad32, p16


def test_fullsize_zero2_7p5b_rank0():
    """7.5B at Nd = 64, rank 0: five buckets (17,187,500 + 4 x 25M), 10 steps."""
    _run_zero2(wl.zero2_7p5b(0))


def _fullstate(w):
    """Every element, not a sample, of one rank's shard in the bench's launch
    configuration: the gradient Adam reads (the reduced fp32 shard after the
    reduce pass over all buckets, or plain data parallelism's raw fp16
    gradient), then master, m, v and the fp16 slot after each of the
    workload's Adam steps.  The oracle runs over the whole shard in
    2^22-element chunks in a spawn pool (tests/oracle_pool.py) while the device
    works, and returns per-chunk SHA-256 digests; the device results are hashed
    the same way after each step.  A chunk that differs is compared element by
    element under the bars of tests/gpu_util.py, from the device state before
    that step (kept as one snapshot), so a failure names the elements."""
    geom = Z.shard_geometry(w.psi, w.nd, w.rank)
    lo, S = geom.offset, geom.len
    print(f"{w.name}: full state over [{lo}, +{S}), {w.steps} steps, oracle on "
          f"{oracle_pool.workers()} processes", flush=True)
    orc = oracle_pool.ShardOracle(w, lo, S, w.steps)
    try:
        state = _state(w, geom)
        if w.fp16_grad:
            grad = torch.empty(S, dtype=torch.int16, device="cuda")
            sdev.fill_grad_rows(grad.view(1, S), w.seed, lo, w.grad.sigma, w.grad.heavy_tail,
                                kind=gen.KIND_GRAD_FULL)
        elif w.grad_shard == "fp16":
            grad = torch.zeros(S, dtype=torch.int16, device="cuda")
            _reduce_all(w, geom, None, grad16=grad)
        else:
            grad = torch.zeros(S, dtype=torch.float32, device="cuda")
            _reduce_all(w, geom, grad)
        p16 = torch.zeros(w.psi, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        spans = orc.chunks
        g_host = grad.cpu().numpy()
        got_g = oracle_pool.chunk_digests(g_host, spans)
        want = orc.result()
    finally:
        orc.close()
    assert set(want) == {("grad", 0)} | {(n, t) for n in oracle_pool.ARRAYS
                                         for t in range(1, w.steps + 1)}

    half = w.fp16_grad or w.grad_shard == "fp16"

    def oracle_grad(j0, n):
        flat = np.arange(lo + j0, lo + j0 + n, dtype=np.uint64)
        if w.fp16_grad:
            return gen.grad_f16(w.seed, 0, flat, w.grad.sigma, w.grad.heavy_tail,
                                kind=gen.KIND_GRAD_FULL)
        g = _oracle_grad(w, flat)
        return g.astype(np.float16).view(np.uint16) if half else g

    spans_d = dict(spans)
    bad = [j0 for j0, h in sorted(want[("grad", 0)].items()) if got_g[j0] != h]
    if bad:
        j0 = bad[0]
        assert_bits(g_host[j0:j0 + spans_d[j0]].view(np.uint16 if half else np.float32),
                    oracle_grad(j0, spans_d[j0]), f"gradient, chunk {j0}")
        pytest.fail(f"gradient digests differ at chunks {bad[:8]}")
    del g_host
    compared = len(spans)
    for t in range(1, w.steps + 1):
        before = [x.clone() for x in state]
        Z.adam_step_shard(geom, *state, grad, p16, 0, w.lr, w.beta1, w.beta2, w.eps, t)
        torch.cuda.synchronize()
        host = [x.cpu().numpy() for x in state]
        host.append(p16[lo:lo + S].cpu().numpy().view(np.uint16))
        bad = []
        for name, a in zip(oracle_pool.ARRAYS, host):
            d = oracle_pool.chunk_digests(a, spans)
            bad += [(j0, name) for j0, h in want[(name, t)].items() if d[j0] != h]
            compared += len(spans)
        if bad:
            j0, name = min(bad)
            n = spans_d[j0]
            g_ref = oracle_grad(j0, n)
            prev = [x[j0:j0 + n].cpu().numpy() for x in before]
            sc = oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, t)
            assert_adam_step((*prev, oadam.grad_f32(g_ref)),
                             tuple(a[j0:j0 + n] for a in host),
                             oadam.step_values(*prev, g_ref, sc), c1=float(sc.c1),
                             b1=float(sc.b1), b2=float(sc.b2), c2=float(sc.c2),
                             what=f"step {t}, chunk {j0}")
            pytest.fail(f"step {t}: digests differ at {sorted(bad)[:8]}")
        del before, host
        print(f"step {t}: {4 * len(spans)} chunk digests equal", flush=True)
    # nothing outside the slot was written
    assert torch.count_nonzero(p16[:lo]).item() == 0
    assert torch.count_nonzero(p16[lo + S:]).item() == 0
    assert compared == len(spans) * (1 + len(oracle_pool.ARRAYS) * w.steps)
    print(f"{compared} chunk digests compared, all equal", flush=True)


@pytest.mark.timeout(900)
def test_fullstate_zero2_7p5b_rank0():
    """Every element of the 7.5B / Nd = 64 rank-0 shard (117,187,500): the reduced
    fp32 gradient over the five buckets and the state after each of 10 steps."""
    _fullstate(wl.zero2_7p5b(0))


@pytest.mark.timeout(900)
def test_fullstate_zero2_7p5b_fp16_shard():
    """The same rank with the fp16 gradient shard of the guide's 2 Psi + 14 Psi / Nd
    accounting: every element of the shard as the reduce rounds it to fp16, and
    the state after each of 10 steps of Adam on it."""
    _fullstate(wl.zero2_7p5b_g16(0))


@pytest.mark.timeout(900)
def test_fullstate_zero2_13b_rank0():
    """Every element of the 13B / Nd = 32 rank-0 shard (406,250,000) with
    heavy-tailed gradients (exact zeros and x100 outliers, so partial sums leave
    the exact range): the reduced fp32 gradient over 17 buckets and the state
    after each of 10 steps."""
    _fullstate(wl.zero2_13b(0))


@pytest.mark.timeout(900)
def test_fullstate_plain_dp_1p4b():
    """Every element of plain data parallelism at 1.4B (Nd = 1, no reduce): the
    fused Adam on the raw fp16 gradient, each of 20 steps."""
    _fullstate(wl.plain_dp_1p4b())


def test_fullsize_zero2_7p5b_rank1():
    """Rank 1: six partial/full buckets; its fp16 slot starts 8 bytes off 16-byte alignment."""
    _run_zero2(wl.zero2_7p5b(1))


def test_fullsize_zero2_100b_rank137():
    """100B at Nd = 400, rank 137: 11 tensor-sized buckets, 400 rows streamed in 2^22-element
    chunks, fp16 vector as a window around the slot, 5 steps."""
    w = wl.zero2_100b(137)
    _run_zero2(w, chunk=w.extra["chunk"], window=w.extra["p16_window"])


def test_fullsize_plain_dp_1p4b():
    """Plain DP (Nd = 1, no reduce), 1.4B: the fused Adam on fp16 gradients, 20 steps."""
    w = wl.plain_dp_1p4b()
    geom = Z.shard_geometry(w.psi, 1, 0)
    state = _state(w, geom)
    g16 = torch.empty(geom.len, dtype=torch.int16, device="cuda")
    sdev.fill_grad_rows(g16.view(1, -1), w.seed, 0, w.grad.sigma, kind=gen.KIND_GRAD_FULL)
    p16 = torch.zeros(w.psi, dtype=torch.int16, device="cuda")
    idx = sample_indices(geom.len, [], N_RANDOM, seed=3)
    g_ref = gen.grad_f16(w.seed, 0, idx.astype(np.uint64), w.grad.sigma,
                         kind=gen.KIND_GRAD_FULL)
    assert_bits(gather(g16, idx).cpu().numpy().view(np.uint16), g_ref, "fp16 gradient")
    before = [x.index_select(0, torch.from_numpy(idx).cuda()).cpu().numpy() for x in state]
    for a, b in zip(before, _host_state(w, idx.astype(np.uint64))):
        assert_bits(a, b, "initial state")
    _steps(w, geom, state, g16, g_ref, p16, 0, idx, w.steps, w.name)


def test_fullsize_zero2_13b_probe():
    """13B at Nd = 32 with heavy-tailed gradients, rank 0 (17 buckets), 10 steps; each step
    the 2^20-element probe straddling ranks 0 and 1 must equal an unsharded step."""
    w = wl.zero2_13b(0)
    probe = w.extra["probe"]
    geom0, state0, grad0, p16 = _run_zero2(w)
    # rank 1 owns the probe's upper half; its gradient shard needs only the bucket
    # that holds those elements, the rest of its shard is never compared
    w1 = wl.zero2_13b(1)
    geom1 = Z.shard_geometry(w1.psi, w1.nd, 1)
    state1 = _state(w1, geom1)
    grad1 = torch.zeros(geom1.len, dtype=torch.float32, device="cuda")
    p_lo, p_hi = geom1.offset - probe // 2, geom1.offset + probe // 2
    for off, n in wl.buckets_touching(w1.buckets, geom1.offset, p_hi):
        a, b = Z.bucket_intersect(geom1, off, n)
        stride = Z.row_stride(b - a)
        buf = torch.empty(w1.nd * stride, dtype=torch.int16, device="cuda")
        rows = buf.as_strided((w1.nd, b - a), (stride, 1))
        sdev.fill_grad_rows(rows, w1.seed, a, w1.grad.sigma, w1.grad.heavy_tail)
        Z.reduce_shard(geom1, a, b - a, rows, grad1)
        del rows, buf
    # the unsharded reference: one rank owning a 2^20-parameter model made of the
    # probe's initial state and reduced gradients
    gu = Z.shard_geometry(probe, 1, 0)
    ref_state = _state_probe(w, p_lo, probe)
    ref_grad = torch.cat([grad0[geom0.len - probe // 2:], grad1[:probe // 2]]).clone()
    # restart both ranks from their initial state (the probe compares trajectories)
    state0 = _state(w, geom0)
    ref_p16 = torch.zeros(probe, dtype=torch.int16, device="cuda")
    for t in range(1, w.steps + 1):
        Z.adam_step_shard(geom0, *state0, grad0, p16, 0, w.lr, w.beta1, w.beta2, w.eps, t)
        Z.adam_step_shard(geom1, *state1, grad1, p16, 0, w.lr, w.beta1, w.beta2, w.eps, t)
        Z.adam_step_shard(gu, *ref_state, ref_grad, ref_p16, 0, w.lr, w.beta1, w.beta2,
                          w.eps, t)
        torch.cuda.synchronize()
        for i in range(3):
            cat = torch.cat([state0[i][geom0.len - probe // 2:], state1[i][:probe // 2]])
            assert torch.equal(cat.view(torch.int32), ref_state[i].view(torch.int32)), (t, i)
        assert torch.equal(p16[p_lo:p_hi], ref_p16), t


def _state_probe(w, lo, n):
    out = []
    for kind, d in ((gen.KIND_MASTER, w.master), (gen.KIND_M, w.m), (gen.KIND_V, w.v)):
        t = torch.empty(n, dtype=torch.float32, device="cuda")
        sdev.fill_state(t, w.seed, kind, lo, d.sigma, d.absolute)
        out.append(t)
    return out


def test_fullsize_zero3_7p5b_rank0():
    """Stage 3 at 7.5B / Nd = 64, rank 0, one step as the bench runs it: every layer
    gathered in forward order, then again in reverse with the owned layer's
    gradient reduced into the fp16 shard, then Adam into the rank's own fp16
    parameter shard.  Sampled against the oracle: a gathered layer crossing two
    other ranks' shards (their generated fp16 parameters), the fp16 gradient
    shard, the state after the step, and a gather after the step that must return
    the updated own shard where the layer crosses it."""
    w = wl.zero3_7p5b(0)
    psi, nd, rank = w.psi, w.nd, w.rank
    geom = Z.shard_geometry(psi, nd, rank)
    lo, S = geom.offset, geom.len
    print(f"{w.name}: shard [{lo}, +{S})", flush=True)
    s_all = -(-psi // nd)
    sigma_p = w.extra["param_sigma"]
    shards = torch.empty((nd, s_all), dtype=torch.int16, device="cuda")
    for k in range(nd):
        k_lo = min(k * s_all, psi)
        k_n = min((k + 1) * s_all, psi) - k_lo
        if k_n:
            sdev.fill_grad_rows(shards[k:k + 1, :k_n], w.seed, k_lo, sigma_p, rank0=k,
                                kind=gen.KIND_PARAM16)
    state = _state(w, geom)
    grad16 = torch.zeros(S, dtype=torch.int16, device="cuda")
    layers = list(reversed(w.buckets))                          # forward order
    layer_buf = torch.empty(max(n for _, n in layers), dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(9)

    def owner_values(flat):
        k = (flat // np.uint64(s_all)).astype(np.int64)
        out = np.empty(flat.size, np.uint16)
        for kk in np.unique(k):
            sel = k == kk
            out[sel] = gen.grad_f16(w.seed, int(kk), flat[sel], sigma_p, kind=gen.KIND_PARAM16)
        return out, k

    # forward: check the layers that cross two shards, neither of them this rank's
    crossing_checked = 0
    for off, n in layers:
        Z.gather_params(psi, nd, off, n, shards, layer_buf[:n])
        if off // s_all >= 2 and (off + n - 1) // s_all == off // s_all + 1:
            torch.cuda.synchronize()
            rel = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                            rng.integers(0, n, 4096)])).astype(np.int64)
            want, _ = owner_values(rel.astype(np.uint64) + np.uint64(off))
            got = layer_buf.index_select(0, torch.from_numpy(rel).cuda()).cpu().numpy()
            assert_bits(got.view(np.uint16), want, f"forward gather of layer at {off}")
            crossing_checked += 1
    assert crossing_checked > 0
    # backward: gather, then reduce the owned part of the layer's gradient
    edges = []
    for off, n in w.buckets:
        Z.gather_params(psi, nd, off, n, shards, layer_buf[:n])
        a, b = Z.bucket_intersect(geom, off, n)
        if a < b:
            edges += [a - lo, b - lo]
            st = Z.row_stride(b - a)
            buf = torch.empty(nd * st, dtype=torch.int16, device="cuda")
            rows = buf.as_strided((nd, b - a), (st, 1))
            sdev.fill_grad_rows(rows, w.seed, a, w.grad.sigma, w.grad.heavy_tail)
            Z.reduce_shard(geom, a, b - a, rows, None, grad16)
            del rows, buf
    torch.cuda.synchronize()
    idx = sample_indices(S, edges, N_RANDOM, seed=21)
    flat = idx.astype(np.uint64) + np.uint64(lo)
    g32 = _oracle_grad(w, flat)
    g16_ref = g32.astype(np.float16).view(np.uint16)
    assert_bits(gather(grad16, idx).cpu().numpy().view(np.uint16), g16_ref, "fp16 gradient shard")
    # Adam into the own shard (row `rank` of the shard buffer, origin = shard offset)
    it = torch.from_numpy(idx).cuda()
    before = [x.index_select(0, it).cpu().numpy() for x in state]
    Z.adam_step_shard(geom, *state, grad16, shards[rank, :S], lo, w.lr, w.beta1, w.beta2,
                      w.eps, 1)
    torch.cuda.synchronize()
    after = [x.index_select(0, it).cpu().numpy() for x in state]
    sc = oadam.scalars(w.lr, w.beta1, w.beta2, w.eps, 1)
    want = oadam.step_values(*before, g16_ref, sc)
    for got, exp, name in zip(after, want[:3], ("master", "m", "v")):
        assert_bits(got, exp, f"{name} after the step")
    p16 = shards[rank, :S].index_select(0, it).cpu().numpy().view(np.uint16)
    assert_bits(p16, want[3], "own fp16 shard after the step")
    # the next gather of the layer that holds the shard's end sees the update
    last = lo + S - 1
    off, n = next((o, k) for o, k in layers if o <= last < o + k)
    Z.gather_params(psi, nd, off, n, shards, layer_buf[:n])
    torch.cuda.synchronize()
    rel = np.unique(np.concatenate([np.clip(np.arange(last - off - 63, last - off + 65), 0, n - 1),
                                    rng.integers(0, n, 4096)])).astype(np.int64)
    fl = rel.astype(np.uint64) + np.uint64(off)
    want_g, owner = owner_values(fl)
    mine = owner == rank
    pos = np.searchsorted(flat, fl[mine])
    known = (pos < flat.size) & (flat[np.minimum(pos, flat.size - 1)] == fl[mine])
    got = layer_buf.index_select(0, torch.from_numpy(rel).cuda()).cpu().numpy().view(np.uint16)
    others = ~mine
    assert_bits(got[others], want_g[others], "gathered elements of other ranks")
    mine_idx = np.flatnonzero(mine)[known]
    assert mine_idx.size > 0
    assert_bits(got[mine_idx], want[3][pos[known]], "gathered elements of the own shard")
