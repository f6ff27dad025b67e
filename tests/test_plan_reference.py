"""Pins for the integer reference of the work list and the offsets scan.

Costs are checked against brute force: a tile's cost must equal the number of
blocks that hold at least one (query, key) pair the attention uses.
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


@pytest.mark.parametrize("kv_pass", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_plan_is_a_sorted_permutation(kv_pass, causal):
    rng = np.random.default_rng(3 + kv_pass + 2 * causal)
    lq = rng.integers(0, 700, size=23)
    lk = rng.integers(0, 900, size=23)
    qo, ko = oracle.exclusive_scan(lq), oracle.exclusive_scan(lk)
    H, TM, TN = 3, 128, 64
    items = oracle.build_plan(qo, ko, H, TM, TN, causal, kv_pass)
    expect = set()
    for b in range(23):
        n = -(-int(lk[b]) // TN) if kv_pass else -(-int(lq[b]) // TM)
        for h in range(H):
            for t in range(n):
                expect.add((b, h, t))
    got = [tuple(int(x) for x in it[:3]) for it in items]
    assert len(got) == len(expect) and set(got) == expect
    keys = [(-min(int(it[3]), P.COST_KEY_CAP - 1), int(it[0]), int(it[1]), int(it[2])) for it in items]
    assert all(keys[i] < keys[i + 1] for i in range(len(keys) - 1))


def test_cost_key_cap_ties_break_by_index():
    # two sequences whose costs exceed the cap share one key and keep b order
    lq = np.array([1, 1])
    lk = np.array([2000 * 64, 1500 * 64])
    items = oracle.build_plan(oracle.exclusive_scan(lq), oracle.exclusive_scan(lk), 1, 64, 64, False)
    assert [int(x) for x in items[:, 0]] == [0, 1]
    assert [int(x) for x in items[:, 3]] == [2000, 1500]


def test_exclusive_scan():
    lens = np.array([3, 0, 5, 1], dtype=np.int32)
    np.testing.assert_array_equal(oracle.exclusive_scan(lens), [0, 3, 3, 8, 9])
    assert oracle.exclusive_scan([]).tolist() == [0]
