"""The streaming probes behind the bench's ceilings do the work they are timed
for: the copy moves every byte, the write stores its pattern everywhere, and the
row read consumes every row (its XOR reaches the key only if all rows were read)."""
import numpy as np
import pytest
import torch

from gpu_util import need_gpu
from synth import probe

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    print(flush=True)


def test_copy_and_write_move_every_byte():
    n = (1 << 20) + 4            # 16-byte multiple, not a multiple of the grid
    src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    for cap in (0, 8, 10):
        dst.zero_()
        probe.copy(src, dst, cap)
        torch.cuda.synchronize()
        assert torch.equal(dst, src)
        probe.write(dst, cap)
        torch.cuda.synchronize()
        assert bool((dst == 0x3C003C00).all())


@pytest.mark.parametrize("nd", [1, 3, 4, 5, 8, 15, 16, 17, 64])
def test_read_rows_reads_every_row(nd):
    cols, stride = 8 * 64 * 3 + 8, 8 * 64 * 3 + 24
    rng = np.random.default_rng(nd)
    host = rng.integers(0, 2**16, size=nd * stride, dtype=np.uint16)
    buf = torch.from_numpy(host.view(np.int16)).cuda()
    rows = buf.as_strided((nd, cols), (stride, 1))
    words = host.reshape(nd, stride)[:, :cols].reshape(nd, cols // 8, 8).view(np.uint32)
    xor = np.bitwise_xor.reduce(np.bitwise_xor.reduce(words, axis=0), axis=1)  # per thread
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    probe.read_rows(rows, sink, 8, key=int(xor[5]))
    torch.cuda.synchronize()
    hits = np.flatnonzero(xor == xor[5])
    assert int(sink.item()) in set(hits.tolist())
    # a key no thread reaches leaves the sink alone
    miss = next(k for k in range(1, 1 << 20) if k not in set(xor.tolist()))
    sink.fill_(-1)
    probe.read_rows(rows, sink, 8, key=miss)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
