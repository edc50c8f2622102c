"""Logical history position -> physical cache row (TEST INFRASTRUCTURE ONLY).

The index-K cache and the latent cache are both stored per token and addressed
by the same positions (page "DeepSeekV3.2之DSA", part 5.2, third point: two
caches aligned by one set of top-k indices), so one mapping serves both.

Two layouts:
* contiguous: sequence ``seq`` occupies rows ``row0[seq] + s``;
* paged: fixed-size blocks of ``block_size`` tokens; position ``s`` of ``seq``
  lives at row ``block_table[seq, s // block_size] * block_size + s % block_size``.
"""

import numpy as np


def phys_rows(seq, positions, *, row0=None, block_table=None, block_size=0):
    """Physical rows for logical positions of one sequence (int64 array)."""
    s = np.asarray(positions, dtype=np.int64)
    if block_size == 0:
        if row0 is None:
            raise ValueError("contiguous layout needs row0")
        return int(np.asarray(row0)[seq]) + s
    bt = np.asarray(block_table, dtype=np.int64)
    blocks = bt[seq, s // block_size]
    return blocks * block_size + (s % block_size)
