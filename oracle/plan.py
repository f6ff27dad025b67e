"""Integer reference for the offsets scan and the longest-first work lists
(test infrastructure only).

Sources: jagged tensors addressed by prefix-sum offsets ("Jagged Flash
Attention (JFA)", section "Definition"); short sequences must not leave compute
units idle ("Why standard FlashAttention falls short"); persistent kernel
scheduling ("Four generations", item 3). The pages give no cost model or order;
the reading used here:

  q pass (forward and the dQ pass): one item per (b, h, t) with t a tile of TM
    query rows, t < ceil(Lq/TM). Its cost is the number of TN-wide key blocks
    it visits: ceil(Lk/TN), or with the causal mask (key j visible to query i
    iff j <= i) ceil(min((t+1)*TM, Lq, Lk) / TN).
  kv pass (the dK/dV pass): one item per (b, h, t) with t a tile of TN keys,
    t < ceil(Lk/TN). Its cost is the number of TM-row query blocks it visits:
    ceil(Lq/TM), or with the causal mask 0 if t*TN >= Lq else
    ceil(Lq/TM) - floor(t*TN/TM).

Order, longest first at two levels. The items of one (b, h) form a group
whose cost is the sum of its items' costs (the same for every h of a
sequence). Groups are ranked by group cost descending, then b, then h. Group
rank g goes to queue snake(g): g mod 2Q < Q ? g mod Q : 2Q-1 - (g mod 2Q),
with Q queues (one per XCD of the GPU, so that the items sharing one (b, h)'s
keys and values run under one L2). Inside a queue, groups follow their rank;
inside a group, items are ordered by cost descending, then t ascending. The
queues are stored one after the other. Items of cost 0 stay in the lists:
they still own outputs that must be written.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

N_QUEUES = 8


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


def snake(g: int, n_queues: int) -> int:
    r = g % (2 * n_queues)
    return r if r < n_queues else 2 * n_queues - 1 - r


def build_plan_queues(q_offsets, kv_offsets, H: int, TM: int, TN: int, causal: bool, kv_pass: bool = False,
                      n_queues: int = N_QUEUES) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Work lists as (items int32 [n, 4] of (b, h, tile, cost) with the queues
    stored one after the other, starts int32 [n_queues], counts int32 [n_queues])."""
    qo = [int(x) for x in q_offsets]
    ko = [int(x) for x in kv_offsets]
    B = len(qo) - 1
    seq_items: List[List[Tuple[int, int]]] = []   # per sequence: (tile, cost) in group order
    seq_cost: List[int] = []
    for b in range(B):
        Lq, Lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if kv_pass:
            n, costf = _cdiv(Lk, TN), kv_tile_cost
        else:
            n, costf = _cdiv(Lq, TM), q_tile_cost
        tiles = [(t, costf(Lq, Lk, t, TM, TN, causal)) for t in range(n)]
        tiles.sort(key=lambda tc: (-tc[1], tc[0]))
        seq_items.append(tiles)
        seq_cost.append(sum(c for _, c in tiles))
    order = sorted(range(B), key=lambda b: (-seq_cost[b], b))
    queues: List[List[Tuple[int, int, int, int]]] = [[] for _ in range(n_queues)]
    g = 0
    for b in order:
        for h in range(H):
            queues[snake(g, n_queues)].extend((b, h, t, c) for t, c in seq_items[b])
            g += 1
    counts = np.array([len(qu) for qu in queues], dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32)
    items = np.array([it for qu in queues for it in qu], dtype=np.int32).reshape(-1, 4)
    return items, starts, counts


def build_plan(q_offsets, kv_offsets, H: int, TM: int, TN: int, causal: bool, kv_pass: bool = False,
               n_queues: int = N_QUEUES) -> np.ndarray:
    """All items, queues concatenated (see build_plan_queues)."""
    return build_plan_queues(q_offsets, kv_offsets, H, TM, TN, causal, kv_pass, n_queues)[0]
