"""CPU checks of the test-side operand layout helper against slots placed by hand.

The layout is libquest's own (declared with ``quest_operand_bytes`` in
include/quest.h), not the pages'; these checks pin the helper that the GPU
product tests use to feed oracle-built operands to the kernel and to read the
operand forward's output back.
"""
import numpy as np

from operand_layout import tile_operand, untile_operand


def test_slot_positions_placed_by_hand():
    # Byte j of run t (columns 32 t .. 32 t + 31) of row r sits at
    # (r // 32) * (C / 128) * 3072 + (t // 4) * 3072 + (t // 2 % 2) * 1536 + (32 (t % 2) + r % 32) * 24 + j.
    rows, cols = 45, 384
    rng = np.random.default_rng(5)
    op = rng.integers(0, 256, size=(rows, cols * 6 // 8), dtype=np.uint8)
    tiled = tile_operand(op, rows, cols)
    assert tiled.size == 64 * cols * 6 // 8
    for r, t, j in [(0, 0, 0), (1, 0, 5), (31, 1, 23), (32, 2, 0), (44, 11, 17), (7, 6, 9), (3, 3, 12)]:
        pos = (r // 32) * (cols // 128) * 3072 + (t // 4) * 3072 + (t // 2 % 2) * 1536 + (32 * (t % 2) + r % 32) * 24 + j
        assert tiled[pos] == op[r, 24 * t + j]


def test_every_byte_lands_once_and_round_trips():
    rows, cols = 70, 256
    op = (np.arange(rows * cols * 6 // 8, dtype=np.int64) % 251 + 1).astype(np.uint8).reshape(rows, -1)
    tiled = tile_operand(op, rows, cols)
    # every byte of the operand appears, and the rest (padding rows) is zero
    assert np.count_nonzero(tiled) == op.size
    assert np.array_equal(np.sort(tiled[tiled != 0]), np.sort(op.reshape(-1)))
    assert np.array_equal(untile_operand(tiled, rows, cols), op)


def test_padding_rows_are_zero():
    rows, cols = 45, 384
    op = np.full((rows, cols * 6 // 8), 0xFF, dtype=np.uint8)
    tiled = tile_operand(op, rows, cols)
    last = tiled[(cols // 128) * 3072:].reshape(cols // 128, 2, 64, 24)
    for rr in range(rows % 32, 32):
        assert not last[:, :, rr, :].any() and not last[:, :, 32 + rr, :].any()
    for rr in range(rows % 32):
        assert last[:, :, rr, :].all() and last[:, :, 32 + rr, :].all()


def test_rejects_bad_shapes():
    import pytest

    with pytest.raises(ValueError):
        tile_operand(np.zeros((4, 72), dtype=np.uint8), 4, 96)
    with pytest.raises(ValueError):
        tile_operand(np.zeros((4, 95), dtype=np.uint8), 4, 128)
