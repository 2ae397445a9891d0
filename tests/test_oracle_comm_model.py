"""Pins of oracle.comm_model and of the K-general memory model.

upskillscore guide "ZeRO: particionar estados do treino entre GPUs", section
"Como funciona": plain DP moves 2 Psi per step (a reduce-scatter and an
all-gather of Psi each), P_os+g the same 2 Psi, P_os+g+p 3 Psi (two parameter
all-gathers and the gradient reduce-scatter), i.e. 1.5x.  lastdictionary entry
"ZeRO": stages 1 and 2 keep data parallelism's volume; stage 3 adds about 50%.
"""
import itertools

import pytest

from oracle import comm_model as cm
from oracle import memory_model as mm


def test_pages_counts():
    psi = 7.5e9
    assert cm.comm_volume(psi, 64, 0).elems == 2 * psi
    assert cm.comm_volume(psi, 64, 1).elems == 2 * psi     # dictionary: same as DP
    assert cm.comm_volume(psi, 64, 2).elems == 2 * psi
    assert cm.comm_volume(psi, 64, 3).elems == 3 * psi
    assert cm.comm_volume(psi, 64, 3).elems / cm.comm_volume(psi, 64, 0).elems == 1.5


def test_collective_kinds():
    assert cm.comm_volume(1, 4, 2).collectives.count("reduce_scatter") == 1
    assert cm.comm_volume(1, 4, 2).collectives.count("all_gather") == 1
    assert cm.comm_volume(1, 4, 3).collectives.count("all_gather") == 2
    assert cm.comm_volume(1, 4, 3).collectives.count("reduce_scatter") == 1


def _ring_reduce_scatter(data):
    """Ring reduce-scatter over nd ranks, simulated: data[r][c] is rank r's chunk
    c (a list of numbers).  At step s rank r sends its running partial of chunk
    (r - s) % nd to rank r + 1, which adds its own.  Returns (the chunk each rank
    ends up owning, elements sent per rank)."""
    nd = len(data)
    part = [[list(ch) for ch in row] for row in data]
    sent = [0] * nd
    for s in range(nd - 1):
        msgs = []
        for r in range(nd):
            c = (r - s) % nd
            msgs.append(((r + 1) % nd, c, part[r][c]))
            sent[r] += len(part[r][c])
        for dst, c, payload in msgs:
            part[dst][c] = [a + b for a, b in zip(part[dst][c], payload)]
    owned = {r: ((r + 1) % nd, part[r][(r + 1) % nd]) for r in range(nd)}
    return owned, sent


def _ring_all_gather(chunks):
    """Ring all-gather: rank r starts with chunk r; at step s it forwards chunk
    (r - s) % nd to rank r + 1.  Returns (what each rank holds, elements sent)."""
    nd = len(chunks)
    have = [{r: chunks[r]} for r in range(nd)]
    sent = [0] * nd
    for s in range(nd - 1):
        msgs = []
        for r in range(nd):
            c = (r - s) % nd
            msgs.append(((r + 1) % nd, c, have[r][c]))
            sent[r] += len(have[r][c])
        for dst, c, payload in msgs:
            have[dst][c] = payload
    return have, sent


def _ring_sent(chunk: int, nd: int, collective: str) -> int:
    """Elements rank 0 sends in a ring collective over a vector of nd chunks,
    after checking that the simulated collective delivers the right result."""
    if collective == "reduce_scatter":
        data = [[[r * 1000 + c * 10 + i for i in range(chunk)] for c in range(nd)]
                for r in range(nd)]
        owned, sent = _ring_reduce_scatter(data)
        for r, (c, vals) in owned.items():
            assert vals == [sum(data[q][c][i] for q in range(nd)) for i in range(chunk)]
        assert sorted(c for c, _ in owned.values()) == list(range(nd))
    else:
        chunks = [[c * 7 + i for i in range(chunk)] for c in range(nd)]
        have, sent = _ring_all_gather(chunks)
        for r in range(nd):
            assert [have[r][c] for c in range(nd)] == chunks
    assert len(set(sent)) == 1                    # every rank sends the same amount
    return sent[0]


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 7, 64])
@pytest.mark.parametrize("stage", [0, 1, 2, 3])
def test_exact_per_rank_volume_by_ring_count(nd, stage):
    chunk = 3
    psi = chunk * nd
    c = cm.comm_volume(psi, nd, stage)
    brute = sum(_ring_sent(chunk, nd, kind) for kind in c.collectives)
    assert c.elems_sent_per_rank == brute
    assert c.bytes_sent_per_rank == 2 * brute


def test_exact_limits():
    psi = 1e9
    assert cm.comm_volume(psi, 1, 0).elems_sent_per_rank == 0
    assert cm.comm_volume(psi, 2, 2).elems_sent_per_rank == psi       # 2 x Psi / 2
    big = 10 ** 9
    assert cm.comm_volume(psi, big, 2).elems_sent_per_rank == pytest.approx(2 * psi, rel=1e-8)
    for nd in (2, 8, 400):
        a = cm.comm_volume(psi, nd, 3).elems_sent_per_rank
        b = cm.comm_volume(psi, nd, 2).elems_sent_per_rank
        assert a / b == pytest.approx(1.5, rel=1e-15)


@pytest.mark.parametrize("nd,stage", [(0, 0), (4, -1), (4, 4)])
def test_comm_bad_args(nd, stage):
    with pytest.raises(ValueError):
        cm.comm_volume(1e9, nd, stage)


# ---- memory model with a general optimizer multiplier K ---------------------------------

def _brute_bytes(psi: int, nd: int, stage: int, k: int, rank: int = 0) -> int:
    """Walk every parameter and count the bytes the device of `rank` keeps for it:
    the fp16 parameter (2 B) unless stage 3 partitions parameters and another
    rank owns it, the fp16 gradient (2 B) unless stage >= 2 and another rank owns
    it, the optimizer state (K B) unless stage >= 1 and another rank owns it."""
    shard = psi // nd
    total = 0
    for i in range(psi):
        mine = i // shard == rank
        total += 2 if (stage < 3 or mine) else 0
        total += 2 if (stage < 2 or mine) else 0
        total += k if (stage < 1 or mine) else 0
    return total


@pytest.mark.parametrize("k", [4, 8, 12, 16])
@pytest.mark.parametrize("nd,stage", list(itertools.product([1, 2, 4, 8], range(4))))
def test_memory_k_brute_force(k, nd, stage):
    psi = 64
    for rank in range(nd):
        assert mm.bytes_per_device(psi, nd, stage, k) == _brute_bytes(psi, nd, stage, k, rank)


@pytest.mark.parametrize("k", [4, 12, 20])
def test_memory_k_limits(k):
    psi, big = 1e9, 10 ** 12
    dp = mm.bytes_per_device(psi, big, 0, k)
    assert dp == (4 + k) * psi
    assert dp / mm.bytes_per_device(psi, big, 1, k) == pytest.approx((4 + k) / 4, rel=1e-9)
    assert dp / mm.bytes_per_device(psi, big, 2, k) == pytest.approx((4 + k) / 2, rel=1e-9)
