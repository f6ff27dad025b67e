"""Moves jagged tensors into and out of the fixed-length slots of the
padded-dense baseline (jfa_fwd_padded / jfa_bwd_padded): sequence b's rows
go to slot b, rows 0 .. L_b - 1, and the rest of the slot is zero. Data
movement only (torch index copies on the device); no attention arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch


def slot_rows(offsets: np.ndarray, slot: int) -> np.ndarray:
    """Row index in the [B * slot] padded layout of every row of the jagged layout."""
    offsets = np.asarray(offsets, dtype=np.int64)
    lengths = np.diff(offsets)
    if len(lengths) and int(lengths.max()) > slot:
        raise ValueError(f"a sequence of {int(lengths.max())} rows does not fit a slot of {slot}")
    seq = np.repeat(np.arange(len(lengths), dtype=np.int64), lengths)
    local = np.arange(int(offsets[-1]), dtype=np.int64) - offsets[:-1][seq] if len(lengths) else np.zeros(0, np.int64)
    return seq * slot + local


def to_slots(x: torch.Tensor, offsets: np.ndarray, slot: int) -> torch.Tensor:
    """[T, ...] jagged -> [B, slot, ...] zero-padded (a new tensor)."""
    B = len(offsets) - 1
    rows = torch.from_numpy(slot_rows(offsets, slot)).to(x.device)
    xp = torch.zeros((B * slot,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    xp[rows] = x
    return xp.view((B, slot) + tuple(x.shape[1:]))


def from_slots(xp: torch.Tensor, offsets: np.ndarray) -> torch.Tensor:
    """[B, slot, ...] padded -> [T, ...] jagged (the rows inside each sequence)."""
    B, slot = xp.shape[0], xp.shape[1]
    rows = torch.from_numpy(slot_rows(offsets, slot)).to(xp.device)
    return xp.reshape((B * slot,) + tuple(xp.shape[2:]))[rows]


def slot_bytes(B: int, q_slot: int, kv_slot: int, H: int, D: int, elt: int = 2) -> int:
    """Device bytes of one padded step's tensors: q, out, dout, dq at [B, q_slot, H, D], lse at
    [B, q_slot, H] fp32, k, v, dk, dv at [B, kv_slot, H, D]."""
    return 4 * B * q_slot * H * D * elt + B * q_slot * H * 4 + 4 * B * kv_slot * H * D * elt


def jagged_bytes(Tq: int, Tk: int, H: int, D: int, elt: int = 2) -> int:
    """The same tensors in the jagged layout."""
    return 4 * Tq * H * D * elt + Tq * H * 4 + 4 * Tk * H * D * elt
