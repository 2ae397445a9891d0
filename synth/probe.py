"""Streaming probes (``synth/libzprobe.so``, from ``synth/csrc/stream_probe.hip``):
plain device reads, writes and copies whose rates are the practical HBM
ceilings reported beside the path's kernels.  They compute nothing of the
method."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzprobe.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        u64, u32, vp, ci = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
        lib.zprobe_read_rows.argtypes = [vp, u64, u32, u64, ci, u32, vp, vp]
        lib.zprobe_read_rows.restype = ci
        lib.zprobe_write.argtypes = [vp, u64, ci, vp]
        lib.zprobe_write.restype = ci
        lib.zprobe_copy.argtypes = [vp, vp, u64, ci, vp]
        lib.zprobe_copy.restype = ci
        lib.zprobe_residency.argtypes = [vp, u32, u32, u32, vp]
        lib.zprobe_residency.restype = ci
        _lib = lib
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _span_ok(t: torch.Tensor, last: int) -> None:
    """Element `last` past t's first element lies inside t's storage."""
    room = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if last >= room:
        raise ValueError("view reaches beyond its storage")


def read_rows(rows: torch.Tensor, sink: torch.Tensor, wgs_per_cu: int = 8,
              key: int = 0x5A5A5A5A, stream=None) -> None:
    """Read an [Nd, cols] int16 view (row stride rows.stride(0)) with the reduce's
    access pattern; sink is a device int32 tensor of one element."""
    if rows.dim() != 2 or rows.dtype != torch.int16 or rows.stride(1) != 1 or not rows.is_cuda:
        raise ValueError("rows must be a 2-D int16 device view with unit column stride")
    if sink.dtype != torch.int32 or sink.numel() < 1 or not sink.is_cuda:
        raise ValueError("sink must be a device int32 tensor")
    nd, cols = rows.shape
    _span_ok(rows, (nd - 1) * rows.stride(0) + cols - 1)
    _check(_load().zprobe_read_rows(rows.data_ptr(), rows.stride(0), nd, cols, wgs_per_cu,
                                    key, sink.data_ptr(), _stream(stream)), "zprobe_read_rows")


def write(dst: torch.Tensor, wgs_per_cu: int = 10, stream=None) -> None:
    if not dst.is_cuda or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous device tensor")
    _check(_load().zprobe_write(dst.data_ptr(), dst.numel() * dst.element_size(), wgs_per_cu,
                                _stream(stream)), "zprobe_write")


def copy(src: torch.Tensor, dst: torch.Tensor, wgs_per_cu: int = 10, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if (not src.is_cuda or not dst.is_cuda or not src.is_contiguous() or
            not dst.is_contiguous() or dst.numel() * dst.element_size() != nbytes):
        raise ValueError("src and dst must be contiguous device tensors of the same size")
    _check(_load().zprobe_copy(src.data_ptr(), dst.data_ptr(), nbytes, wgs_per_cu,
                               _stream(stream)), "zprobe_copy")


def residency(rec: torch.Tensor, blocks: int, lds_bytes: int, sleeps: int = 100,
              stream=None) -> None:
    """Launch `blocks` one-wavefront workgroups with `lds_bytes` of dynamic LDS;
    rec (int64 device tensor of >= 3 * blocks elements) receives per workgroup
    its start and end wall-clock ticks and its compute unit's key."""
    if rec.dtype != torch.int64 or not rec.is_cuda or not rec.is_contiguous() \
            or rec.numel() < 3 * blocks:
        raise ValueError("rec must be a contiguous int64 device tensor of >= 3 * blocks")
    _check(_load().zprobe_residency(rec.data_ptr(), blocks, lds_bytes, sleeps, _stream(stream)),
           "zprobe_residency")


def max_resident(rec) -> dict:
    """From residency()'s records (host int64 [blocks, 3]): the most workgroups
    whose intervals overlap on each compute unit."""
    import numpy as np
    rec = np.asarray(rec).reshape(-1, 3)
    out = {}
    for key in np.unique(rec[:, 2]):
        r = rec[rec[:, 2] == key]
        # ends sort before starts at equal ticks: touching intervals do not overlap
        ev = np.concatenate([np.stack([r[:, 0], np.ones(len(r), np.int64)], 1),
                             np.stack([r[:, 1], -np.ones(len(r), np.int64)], 1)])
        ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
        out[int(key)] = int(np.max(np.cumsum(ev[:, 1])))
    return out
