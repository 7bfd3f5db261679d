"""Exact widening of bfloat16 bit patterns (oracle's own copy; test infrastructure).

A bfloat16 value is the top 16 bits of an IEEE-754 binary32 value, so placing
the 16 bits in the high half of a 32-bit word gives the float32 with the same
value; float32 -> float64 is exact.  No rounding happens anywhere here.
"""
import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 array of bfloat16 bit patterns -> float64 array with identical values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    wide = b.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def as_f64(x):
    """float32/float64 arrays pass through (widened); uint16 arrays are bf16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)
