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

  sq pass (the backward of short-query sequences, Lq <= QMAX = 64, which one
    workgroup owns whole: no dQ pass and no recomputation for them): one item
    per (b, h, c) with c a chunk of TN keys, c < max(1, ceil(Lk/TN)) (a
    sequence without keys still gets one item, which writes its zero dQ). Its
    cost is the number of keys in the chunk, min(TN, Lk - c*TN) (0 if none).
    In the backward, the q and kv passes skip these sequences.

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
SHORT_Q_MAX = 64     # short-query sequences: at most this many queries ...
SHORT_KV_MIN = 1024  # ... and more than this many keys (one chunk of the sq pass)


def short_query(Lq: int, Lk: int) -> bool:
    """Sequences the short-query passes own, split into chunks of keys."""
    return Lq <= SHORT_Q_MAX and Lk > SHORT_KV_MIN


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


def sq_chunk_cost(Lk: int, c: int, TN: int) -> int:
    return max(0, min(TN, Lk - c * TN))


def build_plan_queues(q_offsets, kv_offsets, H: int, TM: int, TN: int, causal: bool, kv_pass: bool = False,
                      n_queues: int = N_QUEUES, kind: str = None, short_q: int = None,
                      with_groups: bool = False):
    """Work lists as (items int32 [n, 4] of (b, h, tile, cost) with the queues
    stored one after the other, starts int32 [n_queues], counts int32 [n_queues]).

    kind: "q", "kv" or "sq" (default: "kv" if kv_pass else "q"). short_q: for
    the q and kv passes, sequences with Lq <= short_q and more than
    SHORT_KV_MIN keys get no items (the sq pass has them).
    with_groups: also return, for the sq pass, int32 [B*H] with the list
    position of chunk 0 of each (b, h) (-1 for sequences the pass skips)."""
    if kind is None:
        kind = "kv" if kv_pass else "q"
    qo = [int(x) for x in q_offsets]
    ko = [int(x) for x in kv_offsets]
    B = len(qo) - 1
    seq_items: List[List[Tuple[int, int]]] = []   # per sequence: (tile, cost) in group order
    seq_cost: List[int] = []
    for b in range(B):
        Lq, Lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if kind == "sq":
            n = _cdiv(Lk, TN) if short_query(Lq, Lk) else 0
            tiles = [(t, sq_chunk_cost(Lk, t, TN)) for t in range(n)]
        else:
            if kind == "kv":
                n, costf = _cdiv(Lk, TN), kv_tile_cost
            else:
                n, costf = _cdiv(Lq, TM), q_tile_cost
            if short_q is not None and Lq <= short_q and Lk > SHORT_KV_MIN:
                n = 0
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
    if not with_groups:
        return items, starts, counts
    first = np.full(B * H, -1, dtype=np.int32)
    for pos, (b, h, t, _) in enumerate(items.tolist()):
        if t == 0:
            first[b * H + h] = pos
    return items, starts, counts, first


def build_plan(q_offsets, kv_offsets, H: int, TM: int, TN: int, causal: bool, kv_pass: bool = False,
               n_queues: int = N_QUEUES) -> np.ndarray:
    """All items, queues concatenated (see build_plan_queues)."""
    return build_plan_queues(q_offsets, kv_offsets, H, TM, TN, causal, kv_pass, n_queues)[0]
