"""The streaming-probe library on the host: it loads, exports its entry points
and rejects bad arguments before any device call (no kernel is launched)."""
import ctypes
import re
import subprocess

from synth import probe


def test_probe_library_exports_and_rejects_bad_arguments():
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert {"zprobe_read_rows", "zprobe_write", "zprobe_copy"} <= \
        set(re.findall(r"\bT (zprobe_[a-z_]+)", out))
    lib = probe._load()
    p16 = ctypes.c_void_p(16)
    sink = ctypes.c_void_p(64)
    # null pointers, zero rows, columns or strides not multiples of 8, stride < cols,
    # misaligned rows, empty grids
    assert lib.zprobe_read_rows(None, 8, 1, 8, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(p16, 8, 1, 8, 8, 0, None, None) == -1
    assert lib.zprobe_read_rows(p16, 8, 0, 8, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(p16, 8, 1, 12, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(p16, 12, 1, 8, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(p16, 8, 1, 16, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(ctypes.c_void_p(18), 8, 1, 8, 8, 0, sink, None) == -1
    assert lib.zprobe_read_rows(p16, 8, 1, 0, 8, 0, sink, None) == -1
    assert lib.zprobe_write(None, 16, 0, None) == -1
    assert lib.zprobe_write(p16, 15, 0, None) == -1
    assert lib.zprobe_write(ctypes.c_void_p(8), 16, 0, None) == -1
    assert lib.zprobe_write(p16, 0, 0, None) == -1
    assert lib.zprobe_copy(None, p16, 16, 0, None) == -1
    assert lib.zprobe_copy(p16, ctypes.c_void_p(32), 17, 0, None) == -1
    assert lib.zprobe_copy(p16, ctypes.c_void_p(32), 32, 0, None) == -1   # overlapping
    assert lib.zprobe_copy(ctypes.c_void_p(24), ctypes.c_void_p(64), 16, 0, None) == -1
