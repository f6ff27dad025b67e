"""Pins for the integer reference of the work lists and the offsets scan.

Costs are checked against brute force: a tile's cost must equal the number of
blocks that hold at least one (query, key) pair the attention uses. The list
order is checked against its stated properties.
"""
import numpy as np
import pytest

import oracle
from oracle import plan as P


def _visible(i, j, causal):
    return (not causal) or j <= i


def _brute_q_cost(Lq, Lk, t, TM, TN, causal):
    rows = range(t * TM, min((t + 1) * TM, Lq))
    blocks = {j // TN for i in rows for j in range(Lk) if _visible(i, j, causal)}
    if not blocks:
        return 0
    # the kernel visits blocks 0 .. max: they are contiguous from 0
    assert blocks == set(range(max(blocks) + 1))
    return max(blocks) + 1


def _brute_kv_cost(Lq, Lk, t, TM, TN, causal):
    keys = range(t * TN, min((t + 1) * TN, Lk))
    blocks = {i // TM for j in keys for i in range(Lq) if _visible(i, j, causal)}
    if not blocks:
        return 0
    lo, hi = min(blocks), max(blocks)
    assert blocks == set(range(lo, hi + 1))
    assert hi == -(-Lq // TM) - 1  # always runs to the last query block
    return hi - lo + 1


@pytest.mark.parametrize("TM,TN", [(16, 16), (32, 64), (64, 32), (128, 64), (64, 128), (48, 80)])
def test_costs_brute_force(TM, TN):
    rng = np.random.default_rng(TM * 1000 + TN)
    for _ in range(60):
        Lq, Lk = int(rng.integers(0, 300)), int(rng.integers(0, 300))
        for causal in (False, True):
            for t in range(-(-Lq // TM)):
                assert P.q_tile_cost(Lq, Lk, t, TM, TN, causal) == _brute_q_cost(Lq, Lk, t, TM, TN, causal)
            for t in range(-(-Lk // TN)):
                assert P.kv_tile_cost(Lq, Lk, t, TM, TN, causal) == _brute_kv_cost(Lq, Lk, t, TM, TN, causal)


def test_snake_deal():
    assert [P.snake(g, 4) for g in range(10)] == [0, 1, 2, 3, 3, 2, 1, 0, 0, 1]
    assert [P.snake(g, 1) for g in range(3)] == [0, 0, 0]


@pytest.mark.parametrize("n_queues", [1, 8])
@pytest.mark.parametrize("kv_pass", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_plan_properties(kv_pass, causal, n_queues):
    rng = np.random.default_rng(3 + kv_pass + 2 * causal + n_queues)
    B, H, TM, TN = 23, 3, 128, 64
    lq = rng.integers(0, 700, size=B)
    lk = rng.integers(0, 900, size=B)
    qo, ko = oracle.exclusive_scan(lq), oracle.exclusive_scan(lk)
    items, starts, counts = oracle.build_plan_queues(qo, ko, H, TM, TN, causal, kv_pass, n_queues)
    # every (b, h, t) exactly once, with its cost
    expect = {}
    for b in range(B):
        n = -(-int(lk[b]) // TN) if kv_pass else -(-int(lq[b]) // TM)
        f = P.kv_tile_cost if kv_pass else P.q_tile_cost
        for h in range(H):
            for t in range(n):
                expect[(b, h, t)] = f(int(lq[b]), int(lk[b]), t, TM, TN, causal)
    got = {(int(a), int(b_), int(c)): int(d) for a, b_, c, d in items}
    assert len(items) == len(expect) and got == expect
    assert counts.sum() == len(items) and starts[0] == 0 and np.all(np.diff(starts) == counts[:-1])
    # group costs: one per sequence; groups are contiguous inside a queue and ranked longest first
    gcost = {}
    for (b, h, t), c in expect.items():
        gcost[b] = gcost.get(b, 0) + c
    order = sorted(range(B), key=lambda b: (-gcost.get(b, 0), b))
    rank = {}
    g = 0
    for b in order:
        for h in range(H):
            rank[(b, h)] = g
            g += 1
    for qi in range(n_queues):
        qu = items[starts[qi]:starts[qi] + counts[qi]]
        groups = []
        for b, h, t, c in qu:
            if not groups or groups[-1] != (b, h):
                groups.append((int(b), int(h)))
        assert len(groups) == len(set(groups)), "a group must be contiguous"
        assert all(P.snake(rank[gr], n_queues) == qi for gr in groups)
        assert [rank[gr] for gr in groups] == sorted(rank[gr] for gr in groups)
        for gr in groups:
            its = [(int(c), int(t)) for b, h, t, c in qu if (b, h) == gr]
            assert its == sorted(its, key=lambda ct: (-ct[0], ct[1]))


def test_exclusive_scan():
    lens = np.array([3, 0, 5, 1], dtype=np.int32)
    np.testing.assert_array_equal(oracle.exclusive_scan(lens), [0, 3, 3, 8, 9])
    assert oracle.exclusive_scan([]).tolist() == [0]


@pytest.mark.parametrize("n_queues", [1, 8])
def test_short_query_pass(n_queues):
    """The sq pass: exactly the sequences with Lq <= 64 and more than 1024
    keys, chunks covering their keys once, group table pointing at chunk 0,
    and the q and kv passes skipping exactly those sequences."""
    rng = np.random.default_rng(7 + n_queues)
    B, H, KC = 40, 3, 1024
    lq = rng.integers(0, 130, size=B)
    lq[:8] = [0, 64, 65, 1, 64, 64, 0, 3]
    lk = rng.integers(0, 5000, size=B)
    lk[:8] = [2000, 1025, 3000, 4096, 1024, 0, 1024, 1025]
    qo, ko = oracle.exclusive_scan(lq), oracle.exclusive_scan(lk)
    items, starts, counts, first = oracle.build_plan_queues(qo, ko, H, 64, KC, False, kind="sq", n_queues=n_queues,
                                                            with_groups=True)
    short = [b for b in range(B) if lq[b] <= 64 and lk[b] > 1024]
    assert {0, 1, 3, 7}.issubset(short) and not {2, 4, 5, 6} & set(short)
    for b in range(B):
        for h in range(H):
            its = [(int(t), int(c)) for bb, hh, t, c in items if bb == b and hh == h]
            if b not in short:
                assert its == [] and first[b * H + h] == -1
                continue
            n = -(-int(lk[b]) // KC)
            assert n >= 2
            assert sorted(t for t, _ in its) == list(range(n))
            assert sum(c for _, c in its) == lk[b]          # the chunks cover every key once
            assert all(c == min(KC, int(lk[b]) - t * KC) for t, c in its)
            pos = first[b * H + h]
            assert tuple(items[pos][:3]) == (b, h, 0)
            assert [tuple(x) for x in items[pos:pos + n, :3]] == [(b, h, t) for t in range(n)]  # contiguous, in order
    for kind, TM, TN in (("q", 128, 64), ("kv", 64, 128)):
        got, _, _ = oracle.build_plan_queues(qo, ko, H, TM, TN, True, kind=kind, short_q=oracle.SHORT_Q_MAX,
                                             n_queues=n_queues)
        full, _, _ = oracle.build_plan_queues(qo, ko, H, TM, TN, True, kind=kind, n_queues=n_queues)
        assert {int(b) for b in got[:, 0]}.isdisjoint(short)
        assert {tuple(x) for x in got.tolist()} == {tuple(x) for x in full.tolist() if x[0] not in short}
