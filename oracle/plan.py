"""Integer reference for the offsets scan and the longest-first work list
(test infrastructure only).

Sources: jagged tensors addressed by prefix-sum offsets ("Jagged Flash
Attention (JFA)", section "Definition"); short sequences must not leave compute
units idle ("Why standard FlashAttention falls short"); persistent kernel
scheduling ("Four generations", item 3). The pages give no cost model or order;
the reading used here is the plainest longest-processing-time-first list:

  q pass (forward and the dQ pass): one item per (b, h, t) with t a tile of TM
    query rows, t < ceil(Lq/TM). Its cost is the number of TN-wide key blocks
    it visits: ceil(Lk/TN), or with the causal mask (key j visible to query i
    iff j <= i) ceil(min((t+1)*TM, Lq, Lk) / TN).
  kv pass (the dK/dV pass): one item per (b, h, t) with t a tile of TN keys,
    t < ceil(Lk/TN). Its cost is the number of TM-row query blocks it visits:
    ceil(Lq/TM), or with the causal mask 0 if t*TN >= Lq else
    ceil(Lq/TM) - floor(t*TN/TM).

Items are ordered by descending cost (cost values at or above COST_KEY_CAP - 1
share one key), then by b, h, t ascending, which makes the order unique.
Items of cost 0 stay in the list: they still own outputs that must be written.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

COST_KEY_CAP = 1024


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def exclusive_scan(lengths) -> np.ndarray:
    """offsets[0] = 0, offsets[b+1] = offsets[b] + lengths[b] (int32)."""
    out = [0]
    for x in lengths:
        out.append(out[-1] + int(x))
    return np.array(out, dtype=np.int64).astype(np.int32)


def q_tile_cost(Lq: int, Lk: int, t: int, TM: int, TN: int, causal: bool) -> int:
    if not causal:
        return _cdiv(Lk, TN)
    return _cdiv(min((t + 1) * TM, Lq, Lk), TN)


def kv_tile_cost(Lq: int, Lk: int, t: int, TM: int, TN: int, causal: bool) -> int:
    nq = _cdiv(Lq, TM)
    if not causal:
        return nq
    first_key = t * TN
    if first_key >= Lq:
        return 0
    return nq - first_key // TM


def build_plan(q_offsets, kv_offsets, H: int, TM: int, TN: int, causal: bool,
               kv_pass: bool = False) -> np.ndarray:
    """Work list as an int32 array [n_items, 4] of (b, h, tile, cost)."""
    qo = [int(x) for x in q_offsets]
    ko = [int(x) for x in kv_offsets]
    items: List[Tuple[int, int, int, int]] = []
    for b in range(len(qo) - 1):
        Lq, Lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if kv_pass:
            n, costf = _cdiv(Lk, TN), kv_tile_cost
        else:
            n, costf = _cdiv(Lq, TM), q_tile_cost
        for h in range(H):
            for t in range(n):
                items.append((b, h, t, costf(Lq, Lk, t, TM, TN, causal)))
    items.sort(key=lambda it: (-min(it[3], COST_KEY_CAP - 1), it[0], it[1], it[2]))
    return np.array(items, dtype=np.int32).reshape(-1, 4)
