"""fp32 -> fp16 round-to-nearest-even written from the IEEE 754 definition in
integer arithmetic, independent of NumPy's cast.  Used only to pin the
oracle's fp16 conversion (the fp16 copy of the reduced gradient and the fp16
parameter slot)."""
import struct


def f32_bits_to_f16_bits(b: int) -> int:
    b = int(b)
    sign = (b >> 31) & 1
    e32 = (b >> 23) & 0xFF
    frac = b & 0x7FFFFF
    s16 = sign << 15
    if e32 == 0xFF:
        return s16 | (0x7E00 if frac else 0x7C00)      # NaN (quiet) or inf
    if e32 == 0:
        if frac == 0:
            return s16
        M, e2 = frac, -149                              # fp32 subnormal: frac * 2^-149
    else:
        M, e2 = frac | 0x800000, e32 - 150              # (2^23 + frac) * 2^(e-150)
    E = M.bit_length() - 1 + e2                         # floor(log2 |x|)
    k = max(E, -14) - 10                                # fp16 quantum exponent at |x|
    if e2 >= k:
        n = M << (e2 - k)
    else:
        sh = k - e2
        n = M >> sh
        rem = M & ((1 << sh) - 1)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and (n & 1)):
            n += 1
    if n == 2048:                                       # rounding carried into the next binade
        n, k = 1024, k + 1
    if n >= 1024:
        field = k + 25
        if field >= 31:
            return s16 | 0x7C00                         # overflow -> inf
        return s16 | (field << 10) | (n - 1024)
    return s16 | n                                      # fp16 subnormal (k == -24)


def f16_bits_to_float(h: int) -> float:
    return struct.unpack("<e", struct.pack("<H", h))[0]


def f32_bits_to_f16_bits_array(bits):
    """The same definition vectorised over a uint32 array (NumPy integer arithmetic
    only, no floating-point cast): returns uint16 fp16 bit patterns."""
    import numpy as np
    b = np.asarray(bits, dtype=np.uint32).astype(np.int64)
    s16 = (b >> 31) << 15
    e = (b >> 23) & 0xFF
    frac = b & 0x7FFFFF
    m = frac | 0x800000                                 # normal significand (2^23 + frac)
    exp = e - 127                                       # floor(log2 |x|) for normal x
    k = np.maximum(exp, -14) - 10                       # fp16 quantum exponent at |x|
    sh = np.minimum(k - (e - 150), 25)                  # >= 13 for every normal fp32 value
    n = m >> sh
    rem = m & ((np.int64(1) << sh) - 1)
    half = np.int64(1) << (sh - 1)
    n = n + ((rem > half) | ((rem == half) & ((n & 1) == 1)))
    carry = n == 2048                                   # rounding into the next binade
    n = np.where(carry, 1024, n)
    k = np.where(carry, k + 1, k)
    field = k + 25
    normal16 = n >= 1024
    out = np.where(normal16, np.where(field >= 31, 0x7C00, (field << 10) | (n - 1024)), n)
    out = np.where(e == 0, 0, out)                      # fp32 subnormals are far below 2^-25
    out = np.where(e == 0xFF, np.where(frac != 0, 0x7E00, 0x7C00), out)
    return (s16 | out).astype(np.uint16)


def f16_bits_of_binade(sign: int, e: int):
    """The definition for every fp32 value with sign `sign` and exponent field
    `e` (all 2^23 significands at once).  The rounding shift is the same for the
    whole binade, so this runs in uint32 arithmetic: n = the significand rounded
    to the fp16 quantum (ties to even); in fp16-normal binades the result is
    n + (k + 24) * 2^10 -- a rounding carry to 2048 lands in the exponent field
    by itself -- clamped to infinity; in fp16-subnormal binades it is n (n = 1024
    there is the smallest normal, 0x0400).  Returns uint16 [2^23]."""
    import numpy as np
    s16 = np.uint32(sign << 15)
    frac = np.arange(1 << 23, dtype=np.uint32)
    if e == 0xFF:
        return (np.where(frac != 0, np.uint32(0x7E00), np.uint32(0x7C00)) | s16).astype(np.uint16)
    if e == 0:                                          # fp32 subnormals: below 2^-25 -> 0
        return np.full(1 << 23, sign << 15, np.uint16)
    m = frac | np.uint32(0x800000)
    exp = e - 127
    k = max(exp, -14) - 10                              # fp16 quantum exponent
    sh = min(k - (e - 150), 25)                         # >= 13
    n = m >> np.uint32(sh)
    rem = m & np.uint32((1 << sh) - 1)
    half = np.uint32(1 << (sh - 1))
    n += ((rem > half) | ((rem == half) & ((n & np.uint32(1)) == 1))).astype(np.uint32)
    if exp >= -14:
        out = np.minimum(n + np.uint32((k + 24) << 10), np.uint32(0x7C00))
    else:
        out = n
    return (out | s16).astype(np.uint16)
