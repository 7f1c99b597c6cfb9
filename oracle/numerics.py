"""Exact widening of the stored element types to fp64 (oracle side).

Test infrastructure only (see the package docstring).

bf16 values are carried as their 16-bit patterns in ``uint16`` arrays.  A bf16
number is the upper half of an IEEE-754 binary32, so shifting the pattern left
by 16 bits yields the binary32 with the same value, which widens to binary64
without rounding.  fp32 widens to fp64 without rounding as well, so every input
the oracle reads is exactly the value the device was given.
"""

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_bits_to_f64(bits):
    """uint16 bf16 patterns -> float64 values, exactly."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bf16 data must be uint16 bit patterns, got {bits.dtype}")
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def to_f64(arr, dtype):
    """Widen stored data of element type ``dtype`` ('f32' or 'bf16') to fp64."""
    if dtype == F32:
        arr = np.asarray(arr)
        if arr.dtype != np.float32:
            raise TypeError(f"f32 data must be float32, got {arr.dtype}")
        return arr.astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(arr)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale_f64(scale):
    """The fp32 scale the device receives, widened exactly."""
    return float(np.float64(np.float32(scale)))
