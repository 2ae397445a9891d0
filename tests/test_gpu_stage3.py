"""Stage 3 (P_os+g+p) on the device through the C ABI, against the oracle.

* zero_gather_params -- the receive side of a layer's parameter all-gather
  (upskillscore guide "ZeRO: particionar estados do treino entre GPUs",
  section "Como funciona"; lastdictionary entry "ZeRO": parameters gathered
  per layer just in time) -- bit for bit against oracle.stage3 over ragged
  ranges, ranges crossing several shards, every relative alignment of source
  and destination, padded shard rows and many small shards;
* a stage-3 step of one rank over a layer schedule: forward gathers of every
  layer, backward gathers with each layer's gradient reduced into the rank's
  gradient shard, then Adam writing the rank's own fp16 shard; two steps, so
  the second step's gathers see the first step's update;
* the device memory that step peaks at: the rank's 16 Psi / Nd, the simulated
  other ranks' shards, and one layer's gathered parameters and gradient rows.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_bits, f32, need_gpu, rows_device, u16
from oracle import adam as oadam
from oracle import geometry as ogeo
from oracle import reduce as ored
from oracle import stage3 as ost3
from synth import device as sdev
from synth import gen, workloads as wl
import zero_sharded_mixed_bucketed_amd as Z
from zero_sharded_mixed_bucketed_amd import rank as zr

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


def _shards_host(psi, nd, width, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 16, size=(nd, width), dtype=np.uint16)


@pytest.mark.parametrize("psi,nd,pad,lo,n,out_shift", [
    (1_000_000, 4, 0, 0, 1_000_000, 0),         # everything: the whole all-gather
    (1_000_000, 4, 0, 249_990, 20, 0),          # across one shard edge
    (1_000_003, 7, 5, 123_457, 700_001, 3),     # several shards, padded rows, odd offsets
    (1_000_003, 7, 1, 142_858, 142_857, 1),     # rows 2 bytes apart: 2-byte copies
    (1_000_003, 7, 2, 3, 500_000, 2),           # 4-byte relative alignment
    (1_000_003, 7, 4, 3, 500_000, 0),           # 8-byte relative alignment
    (600, 200, 0, 5, 590, 0),                   # many small shards: 13 launches of <= 16 pieces
    (1_700, 100, 0, 0, 272, 0),                 # exactly 16 whole shards: one launch
    (1_700, 100, 0, 0, 273, 0),                 # 17 pieces: a second launch of one piece
    (1_700, 100, 3, 5, 267, 1),                 # 16 pieces, ragged at both ends
    (1_700, 100, 3, 5, 268, 1),                 # 17 pieces, ragged at both ends
    (3_300_000, 33, 11, 99_990, 3_000_000, 5),  # 31 pieces of 100,000, lines off by 22 bytes
    (1_000_003, 7, 0, 1_000, 20, 0),            # shorter than the head to the next line
    (10, 3, 0, 9, 1, 1),                        # the last element (short last shard)
])
def test_gather_matches_oracle(psi, nd, pad, lo, n, out_shift):
    print(f"gather psi={psi} nd={nd} pad={pad} lo={lo} n={n} shift={out_shift}", flush=True)
    s = ogeo.shard_size(psi, nd)
    host = _shards_host(psi, nd, s + pad, psi + lo)
    dev = torch.from_numpy(host.view(np.int16)).cuda()
    guard = 40
    base = torch.full((n + 2 * guard + out_shift,), 0x7E01, dtype=torch.int16, device="cuda")
    out = base[guard + out_shift:guard + out_shift + n]
    Z.gather_params(psi, nd, lo, n, dev, out)
    torch.cuda.synchronize()
    assert_bits(u16(out), ost3.gather_params(host, psi, nd, lo, n), "gathered layer")
    b = u16(base)
    assert np.all(b[:guard + out_shift] == 0x7E01) and np.all(b[guard + out_shift + n:] == 0x7E01)


def _oracle_step3(psi, nd, rank, layers, seed, steps, shards0):
    """Oracle of `steps` stage-3 steps of one rank; returns per-step gathered
    layers (forward, step 1 and 2) and the final state."""
    lo, hi = ogeo.shard_range(psi, nd, rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.uint64)
    th = gen.state_f32(seed, gen.KIND_MASTER, idx, 0.02)
    m = gen.state_f32(seed, gen.KIND_M, idx, 1e-4)
    v = gen.state_f32(seed, gen.KIND_V, idx, 1e-6, True)
    shards = shards0.copy()
    gathered = []
    w16 = None
    for t in range(1, steps + 1):
        gathered.append([ost3.gather_params(shards, psi, nd, a, b) for a, b in layers])
        w32 = np.zeros(n, np.float32)
        w16 = np.zeros(n, np.uint16)
        for a, b in reversed(layers):                       # backward, layer by layer
            x, y = ogeo.intersect(lo, hi, a, b)
            if x == y:
                continue
            rows = gen.grad_rows(seed + t, nd, x, y, 1e-3)
            ored.reduce_shard(psi, nd, rank, x, y - x, rows, w32, w16)
        th, m, v, p16 = oadam.step_values(th, m, v, w16, oadam.scalars(LR, B1, B2, EPS, t))
        shards[rank, :n] = p16
    return gathered, w16, th, m, v, shards[rank, :n].copy()


@pytest.mark.parametrize("hidden,layers_n,nd,rank", [(64, 5, 4, 1), (48, 7, 6, 5)])
def test_stage3_step_matches_oracle(hidden, layers_n, nd, rank):
    per = 12 * hidden * hidden + 2 * hidden
    psi = per * layers_n
    print(f"stage3 psi={psi} nd={nd} rank={rank} hidden={hidden}", flush=True)
    seed, steps = 909, 2
    layers = wl.transformer_layers(psi, hidden)
    s = ogeo.shard_size(psi, nd)
    shards0 = np.zeros((nd, s), np.uint16)
    for r in range(nd):                                     # every rank's fp16 shard
        a, b = ogeo.shard_range(psi, nd, r)
        shards0[r, :b - a] = gen.state_f32(seed, gen.KIND_MASTER,
                                           np.arange(a, b, dtype=np.uint64), 0.02) \
            .astype(np.float16).view(np.uint16)
    everyone = torch.from_numpy(shards0.view(np.int16).copy()).cuda()
    st = zr.RankState(psi, nd, rank, 3, param_shard=everyone[rank])
    lo = st.geom.offset
    sdev.fill_state(st.master, seed, gen.KIND_MASTER, lo, 0.02)
    sdev.fill_state(st.m, seed, gen.KIND_M, lo, 1e-4)
    sdev.fill_state(st.v, seed, gen.KIND_V, lo, 1e-6, True)
    want_g, w16, th, m, v, p16 = _oracle_step3(psi, nd, rank, layers, seed, steps, shards0)
    for t in range(1, steps + 1):
        for li, (a, b) in enumerate(layers):                # forward: gather, use, release
            buf = torch.empty(b, dtype=torch.int16, device="cuda")
            st.gather_layer(a, b, everyone, buf)
            torch.cuda.synchronize()
            assert_bits(u16(buf), want_g[t - 1][li], f"step {t} layer {li} forward gather")
            del buf
        for a, b in reversed(layers):                       # backward
            buf = torch.empty(b, dtype=torch.int16, device="cuda")
            st.gather_layer(a, b, everyone, buf)
            x, y = Z.bucket_intersect(st.geom, a, b)
            if x < y:                                       # the owned columns arrive
                rows = rows_device(seed + t, nd, x, y - x, wl.Dist(1e-3))
                st.reduce_bucket(x, y - x, rows)
                del rows
            del buf
        st.adam_step(LR, B1, B2, EPS, t)
    torch.cuda.synchronize()
    assert_bits(u16(st.grad), w16, "gradient shard")
    assert_bits(f32(st.master), th, "master")
    assert_bits(f32(st.m), m, "m")
    assert_bits(f32(st.v), v, "v")
    assert_bits(u16(st.param16), p16, "own fp16 shard")
    others = [k for k in range(nd) if k != rank]
    assert_bits(u16(everyone)[others], shards0[others], "other ranks' shards untouched")


def _r512(nbytes):
    return -(-nbytes // 512) * 512


def test_stage3_peak_memory():
    hidden, layers_n, nd, rank = 64, 8, 4, 2          # shard of 98,560 = 385 x 256 elements
    per = 12 * hidden * hidden + 2 * hidden
    psi = per * layers_n
    layers = wl.transformer_layers(psi, hidden)
    rows_device(1, nd, 0, 256, wl.Dist(1e-3))               # generator tables first
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    s = ogeo.shard_size(psi, nd)
    everyone = torch.zeros((nd, s), dtype=torch.int16, device="cuda")
    st = zr.RankState(psi, nd, rank, 3, param_shard=everyone[rank])
    fixed = torch.cuda.memory_allocated() - base
    worst = 0
    for a, b in reversed(layers):
        buf = torch.empty(b, dtype=torch.int16, device="cuda")
        st.gather_layer(a, b, everyone, buf)
        x, y = Z.bucket_intersect(st.geom, a, b)
        extra = _r512(2 * b)
        if x < y:
            rows = rows_device(7, nd, x, y - x, wl.Dist(1e-3))
            st.reduce_bucket(x, y - x, rows)
            extra += _r512(2 * nd * (y - x))
            del rows
        worst = max(worst, extra)
        del buf
    st.adam_step(LR, B1, B2, EPS, 1)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    own = _r512(2 * s) * 2 + _r512(4 * s) * 3                   # param + grad shard, master/m/v
    assert own == 16 * s                                        # 16 Psi / Nd (sizes are 512-byte multiples)
    assert fixed == _r512(2 * nd * s) - _r512(2 * s) + own      # + the other ranks' shards
    assert peak == fixed + worst
