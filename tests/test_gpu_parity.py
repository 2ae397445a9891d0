"""GPU parity at sizes the oracle finishes in seconds: the HIP path through
the C ABI against the CPU oracle on the same seeded inputs, element by
element, over several tiles and a ragged tail, including the edge cases of
the method (empty and partial bucket/shard intersections, misaligned shard
slots, Nd = 1, trailing empty shards)."""
import numpy as np
import pytest
import torch

import zero_sharded_mixed_bucketed_amd as Z
from gpu_util import (assert_adam_step, assert_bits, f32, need_gpu, rows_device, state_device,
                      state_host, u16)
from oracle import adam as oadam
from oracle import geometry as ogeo
from oracle import reduce as ored
from synth import gen, workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


# --------------------------------------------------------------------------------------
# the shared generator: device side == host side


@pytest.mark.parametrize("nd,lo,n,stride,heavy", [(4, 0, 1000, None, False),
                                                  (3, 12345, 4099, 4101, False),
                                                  (64, 7_499_000_000, 9000, None, False),
                                                  (32, 999, 20003, None, True)])
def test_generator_device_matches_host(nd, lo, n, stride, heavy):
    print(f"gen nd={nd} lo={lo} n={n} stride={stride} heavy={heavy}", flush=True)
    d = wl.Dist(1e-3, heavy_tail=heavy)
    rows = rows_device(77, nd, lo, n, d, stride=stride)
    torch.cuda.synchronize()
    want = gen.grad_rows(77, nd, lo, lo + n, 1e-3, heavy)
    assert_bits(u16(rows), want, "grad rows")
    for kind, dist in ((gen.KIND_MASTER, wl.Dist(0.02)), (gen.KIND_V, wl.Dist(1e-6, True))):
        t = state_device(77, lo, n, dist, kind)
        torch.cuda.synchronize()
        assert_bits(f32(t), state_host(77, np.arange(lo, lo + n, dtype=np.uint64), dist, kind),
                    "state")


# --------------------------------------------------------------------------------------
# reduce


def _reduce_case(psi, nd, rank, buckets, dist, seed, with16=True, stride_pad=0, guard=64,
                 out_shift=0):
    """Reduce every bucket through the ABI and through the oracle; compare all."""
    geom = Z.shard_geometry(psi, nd, rank)
    lo, hi = ogeo.shard_range(psi, nd, rank)
    n = hi - lo
    canary32 = np.float32(-12345.5)
    # guard bands around the output; out_shift moves the shard off 16-byte alignment
    base32 = torch.full((n + 2 * guard + out_shift,), float(canary32), device="cuda")
    base16 = torch.full((n + 2 * guard + out_shift,), 0x7E01, dtype=torch.int16, device="cuda")
    g32 = base32[guard + out_shift:guard + out_shift + n]
    g16 = base16[guard + out_shift:guard + out_shift + n] if with16 else None
    w32 = np.full(n, canary32, np.float32)
    w16 = np.full(n, 0x7E01, np.uint16)
    touching = wl.buckets_touching(buckets, lo, hi)
    others = [b for b in buckets if b not in touching][:1]     # one that misses the shard
    for off, blen in touching + others:
        rows = rows_device(seed, nd, off, blen, dist, stride=blen + stride_pad)
        Z.reduce_shard(geom, off, blen, rows, g32, g16)
        host_rows = gen.grad_rows(seed, nd, off, off + blen, dist.sigma, dist.heavy_tail)
        ored.reduce_shard(psi, nd, rank, off, blen, host_rows, w32, w16 if with16 else None)
        torch.cuda.synchronize()
        del rows                                   # the release of the local gradient
    b32 = f32(base32)
    assert np.all(b32[:guard + out_shift] == canary32) and np.all(b32[guard + out_shift + n:] == canary32)
    assert_bits(f32(g32), w32, "grad32")
    if with16:
        b16 = u16(base16)
        assert np.all(b16[:guard + out_shift] == 0x7E01) and np.all(b16[guard + out_shift + n:] == 0x7E01)
        assert_bits(u16(g16), w16, "grad16")
    return w32


def test_reduce_tiny_zero2():
    """psi = 2^20, Nd = 4, rank 0, one bucket (N(0, 0.01) fp16 gradients)."""
    w = wl.tiny()
    _reduce_case(w.psi, w.nd, w.rank, w.buckets, w.grad, w.seed)


@pytest.mark.parametrize("psi,nd,rank,bucket", [
    (1_000_003, 3, 1, 99_991),       # ragged shard and odd buckets (2-byte row loads)
    (1_000_003, 3, 2, 99_992),       # short last shard, 16-byte row loads
    (3_000_017, 64, 0, 25_000),      # many ranks, shard spans several buckets
    (3_000_017, 64, 63, 25_004),     # 8-byte row loads
    (2_000_000, 5, 4, 333_334),      # 4-byte row loads
    (1 << 20, 1, 0, 100_000),        # Nd = 1: the mean is the gradient itself
    (600_011, 400, 137, 1_504),      # Nd = 400
])
def test_reduce_ragged(psi, nd, rank, bucket):
    print(f"reduce psi={psi} nd={nd} rank={rank} bucket={bucket}", flush=True)
    _reduce_case(psi, nd, rank, wl.uniform_buckets(psi, bucket), wl.Dist(1e-3), 1000 + nd)


def test_reduce_heavy_tail():
    _reduce_case(2_000_003, 32, 7, wl.uniform_buckets(2_000_003, 50_000),
                 wl.Dist(1e-3, heavy_tail=True), 5)


@pytest.mark.parametrize("stride_pad,out_shift", [(1, 0), (2, 1), (4, 0), (0, 1), (0, 2),
                                                  (8, 3), (6, 2)])
def test_reduce_unaligned(stride_pad, out_shift):
    """Row strides that rule out 16-byte loads and outputs off 16-byte alignment."""
    _reduce_case(700_001, 7, 3, wl.uniform_buckets(700_001, 33_336), wl.Dist(0.01), 9,
                 stride_pad=stride_pad, out_shift=out_shift)


@pytest.mark.parametrize("nd", [2, 15, 31, 33, 48, 63, 65, 97])
def test_reduce_row_batches(nd):
    """Nd values whose rows split into every mix of the kernel's load batches
    (full batches of 16, then 8, 4, 2 and 1): the additions must stay in ascending
    rank order."""
    print(f"reduce nd={nd}", flush=True)
    psi = 40_009 * nd
    _reduce_case(psi, nd, nd // 2, wl.uniform_buckets(psi, 17_001), wl.Dist(0.05), 2000 + nd)


@pytest.mark.parametrize("nd,bucket", [(1000, 3_001), (4096, 777)])
def test_reduce_many_ranks(nd, bucket):
    """Thousands of rows per bucket: the row loop, its batches and the 1/Nd scale."""
    print(f"reduce nd={nd} bucket={bucket}", flush=True)
    psi = nd * 2_003
    _reduce_case(psi, nd, nd // 3, wl.uniform_buckets(psi, bucket), wl.Dist(1e-3), 3000 + nd)


def test_reduce_special_values():
    """inf, NaN, fp16 subnormals, -0 and sums beyond the fp16 range, against the
    oracle (NaN compared as NaN, everything else bit for bit)."""
    nd, n = 5, 4099
    rng = np.random.default_rng(11)
    rows = rng.normal(0, 1e-3, size=(nd, n)).astype(np.float16).view(np.uint16)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x0001, 0x8001, 0x03FF, 0x8000, 0x7BFF,
                         0xFBFF, 0x0000], np.uint16)
    for j in range(1000):                      # a special value in some rows of 1000 columns
        mask = rng.random(nd) < 0.4
        rows[mask, j] = rng.choice(specials, size=int(mask.sum()))
    rows[:, 1000] = 0x8000                     # all -0: the mean is +0 (the sum starts at +0)
    rows[:, 1001] = 0x7BFF                     # sum 5 x 65504 (beyond fp16), mean 65504
    rows[:, 1002] = [0x7C00, 0xFC00, 0, 0, 0]  # inf + -inf = NaN
    rows[:, 1003] = 0x0001                     # subnormal sums stay exact
    geom = Z.shard_geometry(n * nd, nd, 0)       # rank 0 owns flat [0, n)
    dev_rows = torch.from_numpy(rows.view(np.int16).copy()).cuda()
    g32 = torch.full((geom.len,), 9.0, device="cuda")
    g16 = torch.zeros((geom.len,), dtype=torch.int16, device="cuda")
    Z.reduce_shard(geom, 0, n, dev_rows, g32, g16)
    torch.cuda.synchronize()
    w32 = np.full(geom.len, 9.0, np.float32)
    w16 = np.zeros(geom.len, np.uint16)
    with np.errstate(all="ignore"):
        ored.reduce_shard(n * nd, nd, 0, 0, n, rows, w32, w16)
    got32, got16 = f32(g32), u16(g16)
    nan32 = np.isnan(got32) & np.isnan(w32)
    assert np.all((got32.view(np.uint32) == w32.view(np.uint32)) | nan32), "grad32"
    nan16 = np.isnan(got16.view(np.float16)) & np.isnan(w16.view(np.float16))
    assert np.all((got16 == w16) | nan16), "grad16"
    assert got32[1000] == 0 and not np.signbit(got32[1000])
    assert got32[1001] == 65504.0 and got16[1001] == 0x7BFF
    assert np.isnan(got32[1002])
    assert got32[1003] == np.float32(5 * 2.0 ** -24) * np.float32(0.2)


def test_reduce_chunking_and_order_invariance():
    psi, nd, rank = 4_000_000, 8, 5
    geom = Z.shard_geometry(psi, nd, rank)
    d = wl.Dist(1e-3)
    outs = []
    for buckets in (wl.uniform_buckets(psi, 123_457),
                    list(reversed(wl.uniform_buckets(psi, 123_457))),
                    wl.uniform_buckets(psi, 1 << 16),
                    [(geom.offset, geom.len)]):
        g32 = torch.zeros(geom.len, device="cuda")
        for off, n in buckets:
            a, b = Z.bucket_intersect(geom, off, n)
            if a == b:
                continue
            rows = rows_device(31, nd, a, b - a, d)     # only the owned columns arrive
            Z.reduce_shard(geom, a, b - a, rows, g32)
        torch.cuda.synchronize()
        outs.append(f32(g32))
    for o in outs[1:]:
        assert_bits(o, outs[0], "chunked/ordered")


def test_reduce_partial_bucket_leaves_rest():
    psi, nd, rank = 1_000_000, 4, 1               # shard [250000, 500000)
    geom = Z.shard_geometry(psi, nd, rank)
    g32 = torch.full((geom.len,), 7.0, device="cuda")
    rows = rows_device(3, nd, 400_001, 150_000, wl.Dist(0.01))
    Z.reduce_shard(geom, 400_001, 150_000, rows, g32)
    torch.cuda.synchronize()
    out = f32(g32)
    assert np.all(out[:150_001] == 7.0)
    host = gen.grad_rows(3, nd, 400_001, 500_000, 0.01)
    assert_bits(out[150_001:], ored.reduce_values(host, nd), "partial")


def test_reduce_empty_and_degenerate():
    geom = Z.shard_geometry(1000, 4, 1)
    g32 = torch.full((geom.len,), 3.0, device="cuda")
    rows = torch.zeros((4, 100), dtype=torch.int16, device="cuda")
    Z.reduce_shard(geom, 0, 100, rows, g32)        # bucket outside the shard
    Z.reduce_shard(geom, 300, 0, rows, g32)        # empty bucket
    z = torch.zeros((4, 1), dtype=torch.int16, device="cuda")
    Z.reduce_shard(geom, 499, 1, z, g32)           # one element: the mean of zeros is +0
    torch.cuda.synchronize()
    out = f32(g32)
    assert np.all(out[:249] == 3.0) and out[249] == 0.0 and not np.signbit(out[249])


# --------------------------------------------------------------------------------------
# Adam


def _adam_case(n, g16, steps, lr, seed, dist_m, dist_v, slot_shift=0, state_shift=0,
               grad_sigma=1e-3, heavy=False):
    """One rank owning n elements (Nd = 1 geometry), per-step comparison."""
    psi = n
    geom = Z.shard_geometry(psi, 1, 0)
    idx = np.arange(n, dtype=np.uint64)
    th_h = gen.state_f32(seed, gen.KIND_MASTER, idx, 0.02)
    m_h = gen.state_f32(seed, gen.KIND_M, idx, dist_m.sigma, dist_m.absolute)
    v_h = gen.state_f32(seed, gen.KIND_V, idx, dist_v.sigma, dist_v.absolute)
    gbits = gen.grad_f16(seed, 0, idx, grad_sigma, heavy_tail=heavy)
    g_h = gbits if g16 else gbits.view(np.float16).astype(np.float32)

    def dev(a, shift):
        base = torch.zeros(n + shift, dtype=torch.float32, device="cuda")
        t = base[shift:]
        t.copy_(torch.from_numpy(a))
        return t
    th, m, v = dev(th_h, state_shift), dev(m_h, state_shift), dev(v_h, state_shift)
    if g16:
        gbase = torch.zeros(n + state_shift, dtype=torch.int16, device="cuda")
        g = gbase[state_shift:]
        g.copy_(torch.from_numpy(gbits.view(np.int16)))
    else:
        g = dev(g_h, state_shift)
    guard = 40
    win = torch.full((n + 2 * guard + slot_shift,), 0x7E01, dtype=torch.int16, device="cuda")
    for t in range(1, steps + 1):
        prev = (th_h, m_h, v_h, g_h if not g16 else gbits.view(np.float16).astype(np.float32))
        Z.adam_step_shard(geom, th, m, v, g, win[guard + slot_shift:], 0, lr, 0.9, 0.999, 1e-8, t)
        torch.cuda.synchronize()
        got = (f32(th), f32(m), f32(v), u16(win)[guard + slot_shift:guard + slot_shift + n])
        want = oadam.step_values(th_h, m_h, v_h, g_h, oadam.scalars(lr, 0.9, 0.999, 1e-8, t))
        sc = oadam.scalars(lr, 0.9, 0.999, 1e-8, t)
        assert_adam_step(prev, got, want, c1=float(sc.c1), b1=float(sc.b1), b2=float(sc.b2),
                         c2=float(sc.c2), what=f"n={n} step {t}")
        w = u16(win)
        assert np.all(w[:guard + slot_shift] == 0x7E01) and np.all(w[guard + slot_shift + n:] == 0x7E01)
        # the next step starts from the GPU's state (identical if bit-exact)
        th_h, m_h, v_h = got[0].copy(), got[1].copy(), got[2].copy()


def test_adam_tiny_zero2():
    """Tiny rank: 262,144 elements, m = v = 0, lr 1e-3, 3 steps, fp32 gradient."""
    _adam_case(262_144, False, 3, 1e-3, wl.SEED_BASE, wl.Dist(0.0), wl.Dist(0.0),
               grad_sigma=0.005)


@pytest.mark.parametrize("n,g16,slot_shift,state_shift", [
    (1_000_003, False, 0, 0),        # ragged tail (n % 4 == 3)
    (1_000_003, True, 0, 0),         # fp16 gradient
    (999_998, True, 1, 0),           # fp16 slot 2 bytes off 4-byte alignment
    (999_998, False, 2, 0),          # slot 4 bytes off 8-byte alignment
    (999_998, False, 4, 0),          # slot 8 bytes off 16-byte alignment
    (500_001, False, 0, 1),          # fp32 arrays off 16-byte alignment: element-wise path
    (500_001, True, 3, 2),
    (1, False, 0, 0),                # one element
    (3, True, 1, 0),
])
def test_adam_ragged_and_misaligned(n, g16, slot_shift, state_shift):
    print(f"adam n={n} g16={g16} slot_shift={slot_shift} state_shift={state_shift}", flush=True)
    _adam_case(n, g16, 3, 1e-4, 4242 + n, wl.Dist(1e-4), wl.Dist(1e-6, True),
               slot_shift=slot_shift, state_shift=state_shift)


def test_adam_plain_dp_like_twenty_steps():
    _adam_case(2_000_000, True, 20, 1e-4, 4243, wl.Dist(1e-4), wl.Dist(1e-6, True))


def test_adam_heavy_tail_zero_moments():
    _adam_case(1_000_000, False, 5, 1e-4, 4244, wl.Dist(0.0), wl.Dist(0.0), heavy=True)


@pytest.mark.parametrize("lr,b1,b2,eps,t", [
    (1e-3, 0.0, 0.999, 1e-8, 1),        # no momentum
    (1e-3, 0.9, 0.0, 1e-8, 2),          # no variance averaging
    (0.0, 0.9, 0.999, 1e-8, 3),         # zero learning rate: the master stays
    (1e-2, 0.9, 0.999, 1.0, 1),         # epsilon dominating the denominator
    (1e-4, 0.9, 0.999, 1e-8, 10 ** 6),  # bias corrections at 1
    (3e-4, 0.5, 0.75, 1e-6, 7),
])
def test_adam_hyperparameter_extremes(lr, b1, b2, eps, t):
    n = 100_003
    geom = Z.shard_geometry(n, 1, 0)
    idx = np.arange(n, dtype=np.uint64)
    th_h = gen.state_f32(77, gen.KIND_MASTER, idx, 0.02)
    m_h = gen.state_f32(77, gen.KIND_M, idx, 1e-4)
    v_h = gen.state_f32(77, gen.KIND_V, idx, 1e-6, True)
    g_h = gen.grad_f16(77, 0, idx, 1e-3).view(np.float16).astype(np.float32)
    th, m, v = (torch.from_numpy(a.copy()).cuda() for a in (th_h, m_h, v_h))
    g = torch.from_numpy(g_h).cuda()
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    Z.adam_step_shard(geom, th, m, v, g, p, 0, lr, b1, b2, eps, t)
    torch.cuda.synchronize()
    sc = oadam.scalars(lr, b1, b2, eps, t)
    want = oadam.step_values(th_h, m_h, v_h, g_h, sc)
    assert_adam_step((th_h, m_h, v_h, g_h), (f32(th), f32(m), f32(v), u16(p)), want,
                     c1=float(sc.c1), b1=float(sc.b1), b2=float(sc.b2), c2=float(sc.c2),
                     what=f"lr={lr} b1={b1} b2={b2} eps={eps} t={t}")
    if lr == 0.0:
        assert_bits(f32(th), th_h, "master with lr = 0")


def test_adam_special_values():
    """Zero gradients from zero moments keep th; inf/NaN gradients propagate."""
    n = 4096
    geom = Z.shard_geometry(n, 1, 0)
    th_h = np.linspace(-1, 1, n, dtype=np.float32)
    g_h = np.zeros(n, np.float32)
    g_h[100] = np.inf
    g_h[101] = np.nan
    g_h[102] = -np.inf
    g_h[103] = 1e30
    g_h[104] = 1e-40                              # fp32 subnormal gradient
    th = torch.from_numpy(th_h.copy()).cuda()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    g = torch.from_numpy(g_h).cuda()
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    Z.adam_step_shard(geom, th, m, v, g, p, 0, 1e-3, 0.9, 0.999, 1e-8, 1)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):      # inf and NaN are the inputs
        want = oadam.step_values(th_h, np.zeros(n, np.float32), np.zeros(n, np.float32), g_h,
                                 oadam.scalars(1e-3, 0.9, 0.999, 1e-8, 1))
    with np.errstate(all="ignore"):
        for got, exp, name in zip((f32(th), f32(m), f32(v), u16(p)), want, "th m v p".split()):
            same = (got.view(np.uint32 if got.dtype == np.float32 else np.uint16) ==
                    exp.view(np.uint32 if exp.dtype == np.float32 else np.uint16))
            nan_both = np.isnan(got.view(np.float32) if got.dtype == np.float32 else
                                got.view(np.float16)) & np.isnan(
                exp.view(np.float32) if exp.dtype == np.float32 else exp.view(np.float16))
            assert np.all(same | nan_both), name
    keep = np.ones(n, bool)
    keep[100:105] = False
    assert np.array_equal(f32(th)[keep], th_h[keep])


# --------------------------------------------------------------------------------------
# sharded == unsharded on the device


@pytest.mark.parametrize("psi,nd", [(1_000_003, 3), (262_147, 8), (100, 16)])
def test_device_sharded_equals_unsharded(psi, nd):
    d_m, d_v = wl.Dist(1e-4), wl.Dist(1e-6, True)
    seed = 606
    flat_u = torch.full((psi,), 0x7E01, dtype=torch.int16, device="cuda")
    flat_s = torch.full((psi,), 0x7E01, dtype=torch.int16, device="cuda")
    gu = Z.shard_geometry(psi, 1, 0)
    full = [state_device(seed, 0, psi, wl.Dist(0.02), gen.KIND_MASTER),
            state_device(seed, 0, psi, d_m, gen.KIND_M),
            state_device(seed, 0, psi, d_v, gen.KIND_V)]
    grad = state_device(seed + 1, 0, psi, wl.Dist(1e-3), gen.KIND_MASTER)
    parts = []
    for r in range(nd):
        g = Z.shard_geometry(psi, nd, r)
        sl = slice(g.offset, g.offset + g.len)
        parts.append((g, [x[sl].clone() for x in full], grad[sl].clone()))
    for t in (1, 2):
        Z.adam_step_shard(gu, *full, grad, flat_u, 0, 1e-4, 0.9, 0.999, 1e-8, t)
        for g, st, gr in parts:
            if g.len == 0:
                continue
            Z.adam_step_shard(g, *st, gr, flat_s, 0, 1e-4, 0.9, 0.999, 1e-8, t)
        torch.cuda.synchronize()
        cat = [torch.cat([p[1][i] for p in parts]) for i in range(3)]
        for a, b in zip(full, cat):
            assert_bits(f32(a), f32(b), "sharded state")
        assert_bits(u16(flat_u), u16(flat_s), "all-gathered fp16 vector")
