"""Host-side logic of bench.py (no GPU): the valid-pair count the throughput is
quoted on, the short/long split, the byte and flop accounting of the roofline
entry, the traffic lines read back from rocprofv3 summaries, and the refusal
of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute_pairs(lq, lk, causal):
    # every (query i, key j) of one sequence; top-left causal alignment keeps j <= i
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return int(np.count_nonzero(j <= i)) if causal else lq * lk


def test_valid_pairs_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(20):
        B = int(rng.integers(1, 12))
        ql = rng.integers(0, 200, size=B)
        kl = rng.integers(0, 200, size=B)
        for causal in (False, True):
            want = sum(_brute_pairs(a, b, causal) for a, b in zip(ql, kl))
            assert bench.valid_pairs(ql, kl, causal) == want


def test_short_long_split_partitions_the_pairs():
    ql = np.array([64, 65, 1, 0, 30, 64, 700])
    kl = np.array([1025, 5000, 1024, 3000, 2000, 1000, 1500])
    for causal in (False, True):
        total = bench.valid_pairs(ql, kl, causal)
        short = bench.valid_pairs(ql, kl, causal, "short")
        long_ = bench.valid_pairs(ql, kl, causal, "long")
        assert short + long_ == total
        # short: at most 64 queries and more than 1024 keys
        sel = (ql <= 64) & (kl > 1024)
        assert short == sum(_brute_pairs(a, b, causal) for a, b in zip(ql[sel], kl[sel]))


class _Wl:
    def __init__(self, H, D, dtype):
        self.H, self.D, self.dtype = H, D, dtype


class _Batch:
    def __init__(self, ql, kl, H, D, dtype="bf16"):
        self.q_lengths, self.kv_lengths = np.array(ql), np.array(kl)
        self.wl = _Wl(H, D, dtype)


def test_algorithmic_bytes():
    b = _Batch([10, 3], [20, 5000], H=2, D=64)  # the second sequence is a short-query one
    e, H, D = 2, 2, 64
    tq, tk, rows = 10 * H * D * e, 20 * H * D * e, 10 * H * 4
    assert bench.algorithmic_bytes("forward", b) == tq + 2 * tk + tq + rows  # q, k, v in; out, lse out
    assert bench.algorithmic_bytes("dkdv", b) == 2 * tq + 2 * tk + 2 * rows + 2 * tk
    assert bench.algorithmic_bytes("dq", b) == 2 * tq + 2 * tk + 2 * rows + tq
    sq, sk = 3 * H * D * e, 5000 * H * D * e
    assert bench.algorithmic_bytes("sq", b) == 3 * sq + 4 * sk + 2 * (3 * H * 4)
    assert bench.algorithmic_bytes("fsq", b) == sq + 2 * sk + sq + 3 * H * 4


def test_flops_per_pair_table():
    # credited: forward QK^T + PV; the backward's 10*D split as dK/dV (S, dP,
    # dV, dK) and dQ (dQ only); the short-query owner forms all five once
    assert bench.KERNEL_FLOPS_PER_PAIR_D == {"forward": 4, "fsq": 4, "dkdv": 8, "dq": 2, "sq": 10}
    assert bench.KERNEL_FLOPS_PER_PAIR_D["dkdv"] + bench.KERNEL_FLOPS_PER_PAIR_D["dq"] == 10
    assert bench.KERNEL_FLOPS_PER_PAIR_D["sq"] == 10
    # executed: the dQ pass recomputes S and dP (4*D) before forming dQ
    assert bench.KERNEL_EXEC_FLOPS_PER_PAIR_D["dq"] == 6


def test_recorded_traffic_reads_matching_lines(tmp_path, monkeypatch):
    src = bench.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x.txt").write_text(
        "  traffic-line kernel=jfa_dq_kernel<bf16,D=64> workload=2 fetch_kib=100.0 write_kib=50.0 "
        f"fetch_scale=2.0 write_scale=1.0 source={src}\n"
        "  traffic-line kernel=jfa_dq_kernel<bf16,D=64> workload=3 fetch_kib=1.0 write_kib=1.0 "
        f"fetch_scale=2.0 write_scale=1.0 source={src}\n"
        "  traffic-line kernel=jfa_fwd_kernel<bf16,D=64> workload=2 fetch_kib=7.0 write_kib=7.0 "
        "fetch_scale=2.0 write_scale=1.0 source=stale\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: src)
    assert bench.recorded_traffic("jfa_dq_kernel<bf16,D=64>", 2) == (100.0 * 2 + 50.0) * 1024
    assert bench.recorded_traffic("jfa_fwd_kernel<bf16,D=64>", 2) is None  # other kernel sources


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
