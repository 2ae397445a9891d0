"""Python binding of libzero: the per-rank data-parallel hot path of ZeRO
stages 1 and 2 on one MI355X.

Argument marshalling only: every step runs in the HIP kernels of libzero.so
(``csrc/``).  Torch tensors supply device memory and the HIP stream.  The
names follow the C ABI in ``include/zero.h``:

    memory_model(psi, nd, stage)                -> bytes per device
    memory_model_k(psi, nd, stage, k)           -> the same with K bytes of optimizer state
    comm_volume(psi, nd, stage)                 -> Comm (collectives and elements per step)
    shard_geometry(psi, nd, rank)               -> Geom
    bucket_intersect(geom, offset, length)      -> (lo, hi)
    reduce_shard(geom, bucket_offset, bucket_len, slices, grad32, grad16=None)
    adam_scalars(lr, beta1, beta2, eps, step)   -> 7 fp32 scalars
    adam_step_shard(geom, master, m, v, grad, param16, param16_origin,
                    lr, beta1, beta2, eps, step)
    gather_params(psi, nd, lo, length, shards, out)
    launch_occupancy(kernel)                    -> (workgroups per CU, dynamic LDS bytes)

Importing this package fails if libzero.so has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero.so")

ZERO_OK = 0
ZERO_E_INVAL = -1
ZERO_E_RANGE = -2
ZERO_E_ALIGN = -3
ZERO_E_DEVICE = -4

STAGE_DP, STAGE_OS, STAGE_OS_G, STAGE_OS_G_P = 0, 1, 2, 3

# Symbols that include/zero.h declares.
EXPORTS = ("zero_memory_model", "zero_memory_model_k", "zero_comm_volume",
           "zero_shard_geometry", "zero_bucket_intersect", "zero_row_stride",
           "zero_reduce_shard", "zero_adam_scalars", "zero_adam_step_shard",
           "zero_gather_params", "zero_launch_occupancy", "zero_last_error")

# Kernels of zero_launch_occupancy.
KERNEL_REDUCE_W16, KERNEL_REDUCE_W8, KERNEL_REDUCE_W4, KERNEL_REDUCE_W2 = 0, 1, 2, 3
KERNEL_ADAM_G32, KERNEL_ADAM_G16 = 4, 5


class ZeroError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libzero error {code}: {msg}")
        self.code = code


class Geom(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_uint64), ("nd", ctypes.c_uint32), ("rank", ctypes.c_uint32),
                ("offset", ctypes.c_uint64), ("len", ctypes.c_uint64)]

    def __repr__(self):
        return (f"Geom(psi={self.psi}, nd={self.nd}, rank={self.rank}, offset={self.offset}, "
                f"len={self.len})")


class Comm(ctypes.Structure):
    _fields_ = [("reduce_scatters", ctypes.c_uint32), ("all_gathers", ctypes.c_uint32),
                ("elems", ctypes.c_double), ("elems_sent_per_rank", ctypes.c_double),
                ("bytes_sent_per_rank", ctypes.c_double)]


class Shard(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("grad", ctypes.c_void_p), ("grad_is_fp16", ctypes.c_int),
                ("param16", ctypes.c_void_p), ("param16_origin", ctypes.c_uint64),
                ("param16_len", ctypes.c_uint64)]


def hip_runtimes() -> set:
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m zero_sharded_mixed_bucketed_amd._build`")
    # torch ships its own HIP runtime; loading torch first makes libzero's
    # libamdhip64.so.7 dependency resolve to that same, already-mapped runtime.
    # Two runtimes in one process would each own the GPU and hand each other
    # pointers they do not know.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    if len(hip_runtimes()) > 1:
        raise ImportError(f"two HIP runtimes are mapped: {sorted(hip_runtimes())}; "
                          "import torch before any other HIP library")
    u64, u32, vp, ci, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int,
                             ctypes.c_double)
    G = ctypes.POINTER(Geom)
    lib.zero_memory_model.argtypes = [u64, u32, ci]
    lib.zero_memory_model.restype = dbl
    lib.zero_memory_model_k.argtypes = [u64, u32, ci, dbl]
    lib.zero_memory_model_k.restype = dbl
    lib.zero_comm_volume.argtypes = [u64, u32, ci, ctypes.POINTER(Comm)]
    lib.zero_comm_volume.restype = ci
    lib.zero_shard_geometry.argtypes = [u64, u32, u32, G]
    lib.zero_shard_geometry.restype = ci
    lib.zero_bucket_intersect.argtypes = [G, u64, u64, ctypes.POINTER(u64), ctypes.POINTER(u64)]
    lib.zero_bucket_intersect.restype = ci
    lib.zero_row_stride.argtypes = [u64, ctypes.POINTER(u64)]
    lib.zero_row_stride.restype = ci
    lib.zero_reduce_shard.argtypes = [G, u64, u64, vp, u64, vp, vp, vp]
    lib.zero_reduce_shard.restype = ci
    lib.zero_adam_scalars.argtypes = [dbl, dbl, dbl, dbl, u64, ctypes.POINTER(ctypes.c_float)]
    lib.zero_adam_scalars.restype = ci
    lib.zero_adam_step_shard.argtypes = [G, ctypes.POINTER(Shard), dbl, dbl, dbl, dbl, u64, vp]
    lib.zero_adam_step_shard.restype = ci
    lib.zero_gather_params.argtypes = [u64, u32, u64, u64, vp, u64, vp, vp]
    lib.zero_gather_params.restype = ci
    lib.zero_launch_occupancy.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(u32)]
    lib.zero_launch_occupancy.restype = ci
    lib.zero_last_error.argtypes = []
    lib.zero_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def last_error() -> str:
    return lib.zero_last_error().decode()


def _check(rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroError(rc, last_error())


def memory_model(psi: int, nd: int, stage: int) -> float:
    """Model-state bytes per device for stage 0 (DP), 1, 2 or 3."""
    b = lib.zero_memory_model(psi, nd, stage)
    if b < 0:
        raise ZeroError(ZERO_E_INVAL, last_error())
    return b


def memory_model_k(psi: int, nd: int, stage: int, k: float) -> float:
    """Model-state bytes per device with K bytes of optimizer state per parameter."""
    b = lib.zero_memory_model_k(psi, nd, stage, k)
    if b < 0:
        raise ZeroError(ZERO_E_INVAL, last_error())
    return b


def comm_volume(psi: int, nd: int, stage: int) -> Comm:
    """Per-step communication of one rank for stage 0 (DP), 1, 2 or 3."""
    c = Comm()
    _check(lib.zero_comm_volume(psi, nd, stage, ctypes.byref(c)))
    return c


def shard_geometry(psi: int, nd: int, rank: int) -> Geom:
    g = Geom()
    _check(lib.zero_shard_geometry(psi, nd, rank, ctypes.byref(g)))
    return g


def bucket_intersect(geom: Geom, offset: int, length: int) -> Tuple[int, int]:
    lo, hi = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.zero_bucket_intersect(ctypes.byref(geom), offset, length, ctypes.byref(lo),
                                     ctypes.byref(hi)))
    return lo.value, hi.value


def row_stride(length: int) -> int:
    """Advised stride (elements) between the Nd gradient rows of `length` columns."""
    out = ctypes.c_uint64()
    _check(lib.zero_row_stride(length, ctypes.byref(out)))
    return out.value


def adam_scalars(lr: float, beta1: float, beta2: float, eps: float, step: int):
    """(b1, b2, c1, c2, eps, step_size, isb) as fp32 values (Python floats)."""
    out = (ctypes.c_float * 7)()
    _check(lib.zero_adam_scalars(lr, beta1, beta2, eps, step, out))
    return tuple(out)


def launch_occupancy(kernel: int, device=None) -> Tuple[int, int]:
    """(workgroups per CU, dynamic LDS bytes) of a capped kernel's launches on
    `device` (default: the current device)."""
    import torch
    wgs, lds = ctypes.c_int(), ctypes.c_uint32()
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    with torch.cuda.device(dev):
        _check(lib.zero_launch_occupancy(kernel, ctypes.byref(wgs), ctypes.byref(lds)))
    return wgs.value, lds.value


def _one_device(tensors, stream):
    """The one device every tensor of a call (and the stream, if given) is on."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"tensors of one call are on {dev} and {t.device}")
    if stream is not None and stream.device != dev:
        raise ValueError(f"the stream is on {stream.device}, the tensors on {dev}")
    return dev


def _launch(tensors, stream, call) -> None:
    """Runs call(stream_handle) with the tensors' device current: the library
    launches on the current device, on the given stream (default: that
    device's current stream)."""
    import torch
    dev = _one_device([t for t in tensors if t is not None], stream)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    handle = ctypes.c_void_p(s.cuda_stream)
    if torch.cuda.current_device() == dev.index:
        _check(call(handle))
    else:
        with torch.cuda.device(dev):
            _check(call(handle))


def _dev(t, name, dtypes, numel_at_least=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel_at_least is not None and t.numel() < numel_at_least:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel_at_least}")


def reduce_shard(geom: Geom, bucket_offset: int, bucket_len: int, slices, grad32,
                 grad16=None, stream=None) -> None:
    """The owner's reduce of one bucket (or chunk) into grad32 and/or grad16.

    slices: int16/float16 device tensor [Nd, >= bucket_len] (row stride =
    slices.stride(0)); row k is rank k's local gradient over the bucket.
    grad32: float32 [geom.len] or None; grad16: int16/float16 [geom.len] or
    None (not both None).  An output may alias a row column for column.
    """
    import torch
    f16 = (torch.int16, torch.float16)
    _dev(slices, "slices", f16)
    if slices.dim() != 2 or slices.shape[0] != geom.nd or slices.stride(1) != 1 \
            or slices.shape[1] < bucket_len:
        raise ValueError("slices must be [Nd, >= bucket_len] with unit column stride")
    if grad32 is None and grad16 is None:
        raise ValueError("grad32 and grad16 are both None")
    if grad32 is not None:
        _dev(grad32, "grad32", (torch.float32,), geom.len)
        if not grad32.is_contiguous():
            raise ValueError("grad32 must be contiguous")
    if grad16 is not None:
        _dev(grad16, "grad16", f16, geom.len)
        if not grad16.is_contiguous():
            raise ValueError("grad16 must be contiguous")
    _launch((slices, grad32, grad16), stream, lambda h: lib.zero_reduce_shard(
        ctypes.byref(geom), bucket_offset, bucket_len, slices.data_ptr(), slices.stride(0),
        grad32.data_ptr() if grad32 is not None else None,
        grad16.data_ptr() if grad16 is not None else None, h))


def adam_step_shard(geom: Geom, master, m, v, grad, param16: Optional[object],
                    param16_origin: int, lr: float, beta1: float, beta2: float, eps: float,
                    step: int, stream=None) -> None:
    """One fused Adam step on the shard; writes the fp16 slot of param16.

    master/m/v: float32 [geom.len], updated in place.  grad: float32, or
    int16/float16 fp16 bits, [geom.len].  param16: int16/float16 window of the
    flat fp16 parameter vector starting at flat index param16_origin, or None.
    """
    import torch
    for name, t in (("master", master), ("m", m), ("v", v)):
        _dev(t, name, (torch.float32,), geom.len)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _dev(grad, "grad", (torch.float32, torch.int16, torch.float16), geom.len)
    if not grad.is_contiguous():
        raise ValueError("grad must be contiguous")
    s = Shard()
    s.master, s.m, s.v = master.data_ptr(), m.data_ptr(), v.data_ptr()
    s.grad = grad.data_ptr()
    s.grad_is_fp16 = 0 if grad.dtype == torch.float32 else 1
    if param16 is not None:
        _dev(param16, "param16", (torch.int16, torch.float16))
        if not param16.is_contiguous():
            raise ValueError("param16 must be contiguous")
        s.param16 = param16.data_ptr()
        s.param16_origin = param16_origin
        s.param16_len = param16.numel()
    _launch((master, m, v, grad, param16), stream, lambda h: lib.zero_adam_step_shard(
        ctypes.byref(geom), ctypes.byref(s), lr, beta1, beta2, eps, step, h))


def gather_params(psi: int, nd: int, lo: int, length: int, shards, out, stream=None) -> None:
    """Stage 3: the fp16 parameters of flat [lo, lo + length) into out, from the
    rank shards (int16/float16 device tensor [Nd, >= S], row k = rank k's
    shard, unit column stride)."""
    import torch
    f16 = (torch.int16, torch.float16)
    _dev(shards, "shards", f16)
    s = -(-psi // nd) if nd > 0 else 0
    if shards.dim() != 2 or shards.shape[0] != nd or shards.stride(1) != 1 \
            or shards.shape[1] < s:
        raise ValueError("shards must be [Nd, >= S] with unit column stride")
    _dev(out, "out", f16, length)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _launch((shards, out), stream, lambda h: lib.zero_gather_params(
        psi, nd, lo, length, shards.data_ptr(), shards.stride(0), out.data_ptr(), h))
