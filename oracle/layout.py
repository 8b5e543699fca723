"""Scale layouts.

A GEMM kernel wants the scales of the rows it works on together; the pages
report that rearranging scales for the GEMM cost more than quantizing
("End-to-End MXFP8 RL on Blackwell", Table 6) and that a stale rearranged copy
was a silent failure (Table 10, F3).  Here the quantizer itself writes the
layout the consumer reads, so no derived copy exists.

LINEAR: the scale grid of a 1D-blocked copy, [rows, blocks_per_row],
row-major.

MFMA (a layout defined by this library, a reading): the grid is cut into
chunks of 32 rows x 4 consecutive blocks; chunks are stored row-chunk-major,
each chunk as 32 little groups of 4 bytes (one per row, its 4 blocks in
order).  Byte offset of (row r, block b) with B = blocks_per_row:
    ((r // 32) * (B // 4) + b // 4) * 128 + (r % 32) * 4 + b % 4
Requires rows % 32 == 0 and B % 4 == 0.

Test infrastructure only (see the package docstring).
"""

import numpy as np


def mfma_offset(r, b, blocks_per_row):
    return ((r // 32) * (blocks_per_row // 4) + b // 4) * 128 + (r % 32) * 4 + b % 4


def linear_to_mfma(scales):
    """Rearrange a LINEAR [rows, B] scale grid into the MFMA byte order."""
    rows, B = scales.shape
    assert rows % 32 == 0 and B % 4 == 0
    out = np.empty(rows * B, dtype=scales.dtype)
    for r in range(rows):
        for b in range(B):
            out[mfma_offset(r, b, B)] = scales[r, b]
    return out


def mfma_to_linear(flat, rows, B):
    out = np.empty((rows, B), dtype=flat.dtype)
    for r in range(rows):
        for b in range(B):
            out[r, b] = flat[mfma_offset(r, b, B)]
    return out
