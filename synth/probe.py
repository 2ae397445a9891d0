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
