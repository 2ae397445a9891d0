"""Pins of oracle.stage3 (upskillscore guide "ZeRO: particionar estados do
treino entre GPUs", section "Como funciona"; lastdictionary entry "ZeRO";
llm-engineer card "ZeRO-2", "Why all-gather is still needed")."""
import numpy as np
import pytest

from oracle import geometry, memory_model, stage3
from synth import workloads as wl


def _shards(psi, nd, seed=0):
    """Rank shards of a random flat fp16 vector, padded rows; returns (flat, shards)."""
    rng = np.random.default_rng(seed)
    flat = rng.integers(0, 1 << 16, size=psi, dtype=np.uint16)
    s = geometry.shard_size(psi, nd)
    shards = np.full((nd, s + 3), 0xDEAD, np.uint16)          # padding never read
    for r in range(nd):
        lo, hi = geometry.shard_range(psi, nd, r)
        shards[r, :hi - lo] = flat[lo:hi]
    return flat, shards


@pytest.mark.parametrize("psi,nd", [(1, 1), (10, 3), (37, 4), (100, 7), (1000, 64)])
def test_all_layers_rebuild_the_vector(psi, nd):
    flat, shards = _shards(psi, nd)
    cuts = sorted({0, psi, *np.random.default_rng(psi).integers(0, psi, 5).tolist()})
    got = np.concatenate([stage3.gather_params(shards, psi, nd, a, b - a)
                          for a, b in zip(cuts[:-1], cuts[1:])])
    assert np.array_equal(got, flat)


@pytest.mark.parametrize("psi,nd", [(10, 3), (37, 4), (100, 7), (65, 8)])
def test_brute_force_owner_scan(psi, nd):
    flat, shards = _shards(psi, nd, 1)
    for lo in range(psi):
        for n in (0, 1, 5, psi - lo):
            if lo + n > psi:
                continue
            got = stage3.gather_params(shards, psi, nd, lo, n)
            for j in range(n):
                i = lo + j
                owner = [r for r in range(nd)
                         if geometry.shard_range(psi, nd, r)[0] <= i < geometry.shard_range(psi, nd, r)[1]]
                assert len(owner) == 1
                r = owner[0]
                assert got[j] == shards[r, i - geometry.shard_range(psi, nd, r)[0]]


def test_rejects_ranges_beyond_psi():
    _, shards = _shards(10, 3)
    with pytest.raises(ValueError):
        stage3.gather_params(shards, 10, 3, 8, 3)


def test_stage3_rank_bytes():
    for psi, nd in ((7_500_000_000, 64), (1 << 20, 4)):
        assert memory_model.bytes_per_device(psi, nd, 3) == 16 * psi / nd


def test_layers_tile_the_vector():
    for psi, h in ((10 ** 11, 8192), (5_000_000, 64), (123_457, 16)):
        layers = wl.transformer_layers(psi, h)
        assert layers[0][0] == 0
        assert all(a + n == b for (a, n), (b, _) in zip(layers, layers[1:]))
        assert layers[-1][0] + layers[-1][1] == psi
        tensors = wl.transformer_tensors(psi, h)
        # every layer boundary is a tensor boundary
        starts = {o for o, _ in tensors}
        assert all(o in starts for o, _ in layers)
