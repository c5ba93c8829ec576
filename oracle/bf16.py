"""bfloat16 conversions for the oracle (test infrastructure only).

bfloat16 is 1 sign + 8 exponent + 7 mantissa bits: the upper half of an
IEEE binary32 ("Quantization basics: from FP32 to INT4", §1.1 floating-point
family and §1.3 format table).  Values are carried as ``uint16`` bit
patterns so that no library rounding is involved on this side.
"""

import numpy as np


def to_f32(bits):
    """Widen bfloat16 bit patterns (uint16 array) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rne(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns uint16 bit patterns.  Subnormals are kept (no flush), overflow
    rounds to +-inf, NaN becomes a quiet NaN with the input's sign.
    The rounding is done on the integer encoding: adding 0x7FFF plus the
    lowest kept bit before truncating the low 16 bits rounds half-way cases
    towards the even neighbour.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(f)
    if np.any(nan):
        sign = (u >> np.uint64(16)).astype(np.uint32) & np.uint32(0x8000)
        rounded = np.where(nan, sign | np.uint32(0x7FC0), rounded)
    return rounded.astype(np.uint16)

