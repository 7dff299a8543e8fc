"""Host-side logic of the QAT linear layer (no GPU): argument checks and defaults."""
from __future__ import annotations

import pytest
import torch

from quantization_aware_amd.linear import GRIDS, ONE_BIT_OUTER_TRUST, QuestLinear, default_trust, quest_linear


def test_grids_listed():
    assert GRIDS == ("int", "fp4", "sparse24")


@pytest.mark.parametrize("grid", ["int8", "", "FP4"])
def test_unknown_grid_rejected(grid):
    with pytest.raises(ValueError):
        QuestLinear(256, 64, grid=grid)
    with pytest.raises(ValueError):
        quest_linear(torch.zeros(2, 256), torch.zeros(4, 256), grid=grid)


def test_trust_defaults():
    # 1.30 for 1-bit operands of the int grid (the pages' s*), 1 otherwise
    assert default_trust(1) == ONE_BIT_OUTER_TRUST == 1.30 and default_trust(4) == 1.0
    layer = QuestLinear(256, 64, bits_x=1, bits_w=2)
    assert layer.trust_x == 1.30 and layer.trust_w == 1.0
    for grid in ("fp4", "sparse24"):
        layer = QuestLinear(256, 64, bits_x=1, bits_w=1, grid=grid)
        assert layer.trust_x == 1.0 and layer.trust_w == 1.0
    assert QuestLinear(256, 64, bits_x=1, trust_x=0.5).trust_x == 0.5


def test_block_must_divide_in_features():
    with pytest.raises(ValueError):
        QuestLinear(200, 64, block=128)


@pytest.mark.parametrize("kw", [dict(grid="fp4"), dict(grid="sparse24"), dict(bits_x=5), dict(bits_w=8)])
def test_freeze_needs_int_grid_and_four_bits(kw):
    # the FP6 product holds midrise levels of at most 4 bits; the check runs before any device work
    with pytest.raises(ValueError):
        QuestLinear(256, 64, **kw).freeze()


def test_train_drops_frozen_operand():
    layer = QuestLinear(256, 64)
    layer._w_operand, layer._w_scale = torch.zeros(1), torch.zeros(1)
    layer.train()
    assert layer._w_operand is None and layer._w_scale is None
