"""The fused step's 16-bit key code, written out in numpy for the tests."""
import numpy as np


def key_code16(u):
    """The fused step's 16-bit key code of order keys u (uint32 array): sign,
    binary exponent clamped to the 16 binades [2^-7, 2^9) (the same field range
    in both halves of the order key), 11 mantissa bits; at least 1."""
    u = np.asarray(u, np.uint32).astype(np.int64)
    s = u >> 31
    f = (u >> 23) & 0xFF
    lo = 127 - 7
    v = ((f - lo) << 11) | ((u >> 12) & 0x7FF)
    v = np.where(f < lo, 0, np.where(f > lo + 15, 0x7FFF, v))
    return np.maximum((s << 15) | v, 1)
