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
