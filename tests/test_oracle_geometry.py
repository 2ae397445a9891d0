"""Pins of oracle.geometry: brute force over tiny models (llm-engineer card
"ZeRO-2", "Why all-gather is still needed": the all-gather of the rank shards
in rank order rebuilds [A, B, C])."""
import pytest

from oracle import geometry as geo


@pytest.mark.parametrize("psi", [1, 2, 7, 12, 13, 37, 100, 1 << 10])
@pytest.mark.parametrize("nd", [1, 2, 3, 4, 5, 8, 13])
def test_shards_partition_the_vector(psi, nd):
    owner = [None] * psi
    prev_hi = 0
    for r in range(nd):
        lo, hi = geo.shard_range(psi, nd, r)
        assert lo == prev_hi            # rank-major and contiguous
        assert hi - lo <= -(-psi // nd)
        for i in range(lo, hi):
            assert owner[i] is None
            owner[i] = r
        prev_hi = hi
    assert prev_hi == psi
    assert all(o is not None for o in owner)


def test_printed_shard_sizes():
    assert geo.shard_size(1 << 20, 4) == 262_144
    assert geo.shard_size(7_500_000_000, 64) == 117_187_500
    assert geo.shard_size(13_000_000_000, 32) == 406_250_000
    assert geo.shard_size(100_000_000_000, 400) == 250_000_000
    assert geo.shard_range(100_000_000_000, 400, 137) == (34_250_000_000, 34_500_000_000)


def test_intersect():
    assert geo.intersect(10, 20, 0, 5) == (10, 10)
    assert geo.intersect(10, 20, 5, 10) == (10, 15)
    assert geo.intersect(10, 20, 12, 3) == (12, 15)
    assert geo.intersect(10, 20, 15, 100) == (15, 20)
    assert geo.intersect(10, 20, 20, 5) == (20, 20)


def test_bad_rank():
    with pytest.raises(ValueError):
        geo.shard_range(10, 2, 2)
    with pytest.raises(ValueError):
        geo.shard_size(10, 0)
