"""Exact bf16 decode (TEST INFRASTRUCTURE ONLY, see the package docstring).

A bf16 value is the upper half of an IEEE fp32 word, so the decode is the
16-bit pattern shifted into the high half of a 32-bit word, read as fp32 and
widened to float64 (exact).
"""

import numpy as np


def bf16_decode(bits):
    """uint16 (or int16) bf16 bit patterns -> float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
