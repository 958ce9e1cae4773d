"""bfloat16 bit helpers for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32 word: 1 sign bit,
8 exponent bits, 7 fraction bits.  numpy has no bfloat16 dtype, so the oracle
holds bf16 tensors as ``uint16`` bit patterns and widens them exactly.
"""

import numpy as np


def to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly (append 16 zero bits)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    return to_f32(bits).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16, ties to even; return uint16 bits.

    Written from the definition: keep the upper 16 bits, and add one unit in
    the last kept place when the dropped 16 bits exceed half a unit, or equal
    exactly half a unit and the kept part is odd.  NaN stays NaN (quiet bit set).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = upper + round_up.astype(np.uint64)
    nan = np.isnan(x)
    out = np.where(nan, (upper | np.uint64(0x40)), out)
    return out.astype(np.uint16)
