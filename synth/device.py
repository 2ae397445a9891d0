"""Device-side generation of the seeded synthetic inputs (torch tensors).

Thin ctypes wrapper over ``synth/libzsynth.so`` (built from
``synth/csrc/synth_gen.hip``).  The values are bit-identical to
``synth.gen`` at the same (seed, kind, rank, flat index).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzsynth.so")
_lib = None
_tables = {}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        # torch (imported above) has mapped its HIP runtime; this library's
        # libamdhip64.so.7 dependency resolves to it.
        lib = ctypes.CDLL(LIB_PATH)
        with open("/proc/self/maps") as f:
            runtimes = {line.split()[-1] for line in f if "libamdhip64" in line}
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are mapped: {sorted(runtimes)}")
        u64, u32, vp, ci = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
        lib.zsynth_grad_rows.argtypes = [vp, u64, u32, u64, u32, u32, u64, u64, vp, vp, ci, vp]
        lib.zsynth_grad_rows.restype = ci
        lib.zsynth_state.argtypes = [vp, u64, u32, u64, u64, vp, vp]
        lib.zsynth_state.restype = ci
        _lib = lib
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _table(key, maker, dtype, device):
    k = (key, dtype, str(device))
    if k not in _tables:
        host = maker()
        _tables[k] = torch.from_numpy(np.array(host, copy=True).view(
            np.int16 if dtype == torch.int16 else np.float32)).to(device)
    return _tables[k]


def fill_grad_rows(out: torch.Tensor, seed: int, lo: int, sigma: float,
                   heavy_tail: bool = False, rank0: int = 0,
                   kind: int = gen.KIND_GRAD) -> None:
    """Fill a [rows, >=len] int16 tensor: row k = rank rank0+k over [lo, lo+len).

    The length is out.shape[1]; a row stride larger than the length is allowed
    through a strided view (out.stride(0) >= out.shape[1]).
    """
    if out.dtype not in (torch.int16, torch.float16) or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be a 2-D row-major int16/float16 tensor")
    rows, n = out.shape
    dev = out.device
    t = _table(("f16", sigma), lambda: gen.table_f16(sigma), torch.int16, dev)
    tail = _table(("f16", sigma * gen.TAIL_SCALE),
                  lambda: gen.table_f16(sigma * gen.TAIL_SCALE), torch.int16, dev)
    rc = _load().zsynth_grad_rows(out.data_ptr(), out.stride(0), rows, seed, kind, rank0,
                                  lo, n, t.data_ptr(), tail.data_ptr(), int(heavy_tail),
                                  _stream())
    if rc != 0:
        raise RuntimeError(f"zsynth_grad_rows failed ({rc})")


def fill_state(out: torch.Tensor, seed: int, kind: int, lo: int, sigma: float,
               absolute: bool = False) -> None:
    """Fill a contiguous fp32 tensor with state stream `kind` over [lo, lo+numel)."""
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor")
    if sigma == 0.0:
        out.zero_()
        return
    t = _table(("f32", sigma, absolute), lambda: gen.table_f32(sigma, absolute),
               torch.float32, out.device)
    rc = _load().zsynth_state(out.data_ptr(), seed, kind, lo, out.numel(), t.data_ptr(),
                              _stream())
    if rc != 0:
        raise RuntimeError(f"zsynth_state failed ({rc})")
