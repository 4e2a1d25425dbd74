"""Rounding of float64 values to bfloat16 (test infrastructure only).

bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the float32
exponent range.  A value is rounded to the nearest representable one, ties
to the even significand; this is done directly from float64 so there is no
double rounding through float32.
"""
import numpy as np


def round_bf16(x):
    """Nearest bfloat16 value of each element of x (ties to even), as float64.

    Values in the normal bf16 range only (the attention operands here are O(1)
    to O(100)); zeros pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    scale = np.ldexp(1.0, e - 8)           # one unit in the 8th significant bit
    # x / scale is exact (power-of-two scaling); np.round rounds half to even
    y = np.round(x / scale) * scale
    return np.where(x == 0.0, 0.0, y)
