"""Exact conversion of stored element formats to float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

bfloat16 values are held as raw ``uint16`` bit patterns: the upper half of an
IEEE-754 binary32. Placing the 16 bits in the high half of a 32-bit word and
reading that word as float32 gives the exact value, which float64 then holds
exactly. float32 arrays widen to float64 exactly.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of each bfloat16 bit pattern (NaN stays NaN)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bfloat16 data must be uint16 bit patterns, got {bits.dtype}")
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """float64 view of a stored array: uint16 = bfloat16 bits, uint8 = FP8 E4M3 bytes (unscaled),
    float32/float64 as is."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    if a.dtype == np.uint8:
        from .fp8 import e4m3_bits_to_f64
        return e4m3_bits_to_f64(a)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported element format {a.dtype}")
