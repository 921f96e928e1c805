"""Exact widening of stored cache values to float64 (oracle; test infrastructure).

A bfloat16 value is the upper half of an IEEE binary32 word, so its bit
pattern shifted left by 16 is the binary32 word of the same value, and every
binary32 value is exactly representable in binary64.  bf16 arrays are held as
``uint16`` bit patterns; float32 arrays are taken as they are.
"""

import numpy as np


def widen(values, dtype):
    """Return ``values`` as float64, exactly.

    ``dtype`` names how ``values`` is stored: ``"f32"`` for float32 arrays,
    ``"bf16"`` for uint16 arrays holding bfloat16 bit patterns, ``"f64"`` for
    float64 arrays (returned as they are; used by pins on float64 inputs).
    """
    a = np.asarray(values)
    if dtype == "f64":
        if a.dtype != np.float64:
            raise TypeError(f"f64 data must be float64, got {a.dtype}")
        return a
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError(f"f32 data must be float32, got {a.dtype}")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError(f"bf16 data must be uint16 bit patterns, got {a.dtype}")
        word = a.astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
            return word.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
