"""Host-side checks of the padded-dense baseline's slot layout (CPU tensors)."""
import numpy as np
import pytest
import torch

from variable_length_attention_jfa_amd import padded


def test_slot_rows_and_round_trip():
    lengths = np.array([3, 0, 5, 1])
    off = np.concatenate([[0], np.cumsum(lengths)])
    rows = padded.slot_rows(off, 6)
    assert rows.tolist() == [0, 1, 2, 12, 13, 14, 15, 16, 18]
    x = torch.arange(9 * 2, dtype=torch.float32).view(9, 2) + 1
    xp = padded.to_slots(x, off, 6)
    assert xp.shape == (4, 6, 2)
    assert torch.all(xp[1] == 0) and torch.all(xp[0, 3:] == 0) and torch.all(xp[3, 1:] == 0)
    assert torch.equal(xp[2, :5], x[3:8])
    assert torch.equal(padded.from_slots(xp, off), x)


def test_slot_too_short_rejected():
    with pytest.raises(ValueError):
        padded.slot_rows(np.array([0, 4, 11]), 6)


def test_byte_ratio():
    # equal slots and lengths: no padding, ratio 1
    assert padded.slot_bytes(4, 8, 8, 2, 64) == padded.jagged_bytes(32, 32, 2, 64)
    assert padded.slot_bytes(4, 16, 16, 2, 64) == 2 * padded.jagged_bytes(32, 32, 2, 64)
