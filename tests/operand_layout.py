"""Test-side helper: the tiled storage layout of libquest's matrix-core operand.

This is a storage format of the library, not part of the method, so it lives
with the tests and not in the oracle.  The layout is the one declared beside
``quest_operand_bytes`` in ``include/quest.h``: rows form blocks of 32 (the
last block padded), each row block is cols/128 consecutive 3072-byte blocks
of 128 columns, a block is two 1536-byte halves of 64 columns, each 64 slots
of 24 bytes; slot l of half e of block c of row block R holds the 32 six-bit
fields of row 32 R + l % 32, columns 128 c + 64 e + 32 (l // 32) .. + 31.

The oracle works on row-major LSB-first 6-bit streams (``operand_e2m3``);
these two functions only move those bytes to and from the tiled layout, so
that the GPU product can be fed operands the oracle built and the GPU
operand forward can be read back.
"""
from __future__ import annotations

import numpy as np

SLOT_BYTES = 24  # 32 fields of 6 bits
BLOCK_BYTES = 3072  # 32 rows x 128 columns x 6 bits


def _slots(rows: int, cols: int):
    """(row, first byte within the row-major row, flat offset) of every slot."""
    rblocks = (rows + 31) // 32
    chunks = cols // 128
    for rb in range(rblocks):
        for c in range(chunks):
            for e in range(2):
                for lane in range(64):
                    row = 32 * rb + lane % 32
                    first_col = 128 * c + 64 * e + 32 * (lane // 32)
                    flat = ((rb * chunks + c) * 2 + e) * 64 * SLOT_BYTES + lane * SLOT_BYTES
                    yield row, first_col * 6 // 8, flat


def tile_operand(op: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Row-major operand (rows x cols*6/8 bytes, cols a multiple of 128) -> flat tiled bytes.

    The padding rows of the last row block are zero.  Returns
    ceil(rows / 32) * 32 * cols * 6 / 8 bytes.
    """
    op = np.asarray(op, dtype=np.uint8)
    if cols % 128 != 0 or op.shape != (rows, cols * 6 // 8):
        raise ValueError("operand must be rows x cols*3/4 bytes with cols a multiple of 128")
    out = np.zeros(((rows + 31) // 32) * 32 * cols * 6 // 8, dtype=np.uint8)
    for row, first, flat in _slots(rows, cols):
        if row < rows:
            out[flat:flat + SLOT_BYTES] = op[row, first:first + SLOT_BYTES]
    return out


def untile_operand(tiled: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Inverse of ``tile_operand``: the row-major rows x cols*6/8 operand (padding dropped)."""
    tiled = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    out = np.zeros((rows, cols * 6 // 8), dtype=np.uint8)
    for row, first, flat in _slots(rows, cols):
        if row < rows:
            out[row, first:first + SLOT_BYTES] = tiled[flat:flat + SLOT_BYTES]
    return out
