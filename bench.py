"""Benchmark: jagged attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N] [--also LIST] [--no-cpu-baseline]

One step is the whole hot path over one synthetic batch already resident in
HBM: jfa_fwd (work-list build + forward kernel) then jfa_bwd (three work
lists and Delta in one launch, dK/dV pass, dQ pass, and for sequences of at
most 64 queries the short-query backward and its dQ sum). Throughput counts valid (query, key) pairs only:
forward 4*D*H*pairs flops, backward 10*D*H*pairs flops (pairs = sum Lq*Lk, or
sum_i min(i+1, Lk) with the causal mask).

Prints one JSON line. `value` is fwd+bwd TFLOP/s of the default workload
(B=64 sequences, lengths uniform in [1, 1024], H=8, D=64, bf16). The
`roofline` entry is for the kernel with the largest share of the step,
timed with HIP events around each of its launches on its own stream over the
timed steps; `cpu_baseline` times the fp64 CPU oracle on a bounded sample of
the same workload on the host cores; `padded_baseline` runs the same batch
copied into zeroed slots of the longest sequence's length through the
library's padded-dense kernels (a -inf key mask on every block, every block
visited) and gives the jagged path's speedup and memory ratio over it;
`cold_cache` times single steps after a 512 MiB write that empties the L2
and Infinity Cache (median, p10, p90), next to the warm back-to-back `value`.
Before the declared warm-up steps, untimed steps run for --prewarm-ms of wall
time so that the clocks have settled whatever --warmup the caller gives
(recorded as `prewarm`). `other_workloads` holds the same figures for the
other four workloads (each with its own roofline entry: HBM GB/s for the
asymmetric short-query workload, MFMA for the others; padded-dense baseline
for the bf16 ones).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0
SHORT_Q_MAX = 64            # sequences with at most this many queries ...
SHORT_KV_MIN = 1024         # ... and more than this many keys take the short-query passes


def valid_pairs(q_lengths, kv_lengths, causal, which="all"):
    """Valid (query, key) pairs per head. which: "all", "long" (sequences the
    query-tile forward and the split backward handle) or "short" (at most
    SHORT_Q_MAX queries and more than SHORT_KV_MIN keys: the short-query
    forward and backward)."""
    total = 0
    for lq, lk in zip(q_lengths.tolist(), kv_lengths.tolist()):
        short = lq <= SHORT_Q_MAX and lk > SHORT_KV_MIN
        if which == "long" and short or which == "short" and not short:
            continue
        if causal:
            m = min(lq, lk)
            total += m * (m + 1) // 2 + (lq - m) * lk
        else:
            total += lq * lk
    return total


def kernel_source_hash() -> str:
    """Hash of the kernel and header sources (the one the study builds are stamped
    with); HBM byte counts recorded for other sources are stale."""
    from variable_length_attention_jfa_amd import build
    return build.source_hash()[:12]


def recorded_traffic(kernel_label: str, workload: int):
    """HBM bytes per launch from the committed rocprofv3 summaries (FETCH_SIZE and
    WRITE_SIZE, scaled by the plain-copy calibration), or None if none matches the
    current kernel sources."""
    import glob
    import re
    src = kernel_source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        with open(path) as fh:
            for line in fh:
                if "traffic-line" not in line:
                    continue
                kv = dict(re.findall(r"(\w+)=(\S+)", line))
                if kv.get("kernel") == kernel_label and kv.get("workload") == str(workload) and kv.get("source") == src:
                    return (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                            float(kv["write_kib"]) * float(kv["write_scale"])) * 1024.0
    return None


# Algorithmic flops per valid pair per head, as multiples of D, credited to
# each kernel: the backward's 10*D (QK^T recomputed once, dP = dO V^T, dV, dK,
# dQ) is split as dK/dV pass 8*D (QK^T, dP, dV, dK) and dQ pass 2*D (dQ); the
# dQ pass also executes QK^T and dP again (4*D more), which is recompute the
# split design adds and is not counted (KERNEL_EXEC_FLOPS_PER_PAIR_D).
KERNEL_FLOPS_PER_PAIR_D = {"forward": 4, "fsq": 4, "dkdv": 8, "dq": 2, "sq": 10}
KERNEL_EXEC_FLOPS_PER_PAIR_D = {"forward": 4, "fsq": 4, "dkdv": 8, "dq": 6, "sq": 10}
KERNEL_SEQS = {"forward": "long", "fsq": "short", "dkdv": "long", "dq": "long", "sq": "short"}


def cold_cache_steps(step, n, torch, flush_mib=512):
    """Per-step times with the caches emptied before each step: a write of
    flush_mib MiB (more than the 4 MB L2 of each XCD plus the 256 MB Infinity
    Cache) outside the events, then one step between two events on the
    current stream. Returns (median, p10, p90) in ms."""
    buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    times = []
    for i in range(n):
        buf.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del buf
    t = np.sort(np.array(times))
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def prewarm(step, torch, min_ms):
    """Runs steps until at least min_ms of wall time has passed (the clocks
    ramp up over the first tens of milliseconds of back-to-back work).
    Returns (steps run, milliseconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            el = (time.perf_counter() - t0) * 1e3
            if el >= min_ms:
                return n, el


def run_workload(idx, steps, warmup, torch, jfa, gen, with_cpu=False, seed=None, bias_grad=False, padded_steps=0,
                 cold_steps=0, prewarm_ms=0.0):
    wl = gen.WORKLOADS[idx]
    batch = gen.make_batch(wl, seed=seed)
    dev = torch.device("cuda")

    def t(vals, bits):
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(vals).to(dev)

    q, k, v = t(batch.q, batch.q_bits), t(batch.k, batch.k_bits), t(batch.v, batch.v_bits)
    do = t(batch.dout, batch.dout_bits)
    qo = torch.from_numpy(batch.q_offsets).to(dev)
    ko = torch.from_numpy(batch.kv_offsets).to(dev)
    bias = None if batch.bias is None else torch.from_numpy(batch.bias).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((batch.total_q, wl.H), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    # the longest key side, known on the host as in a training loop's batch
    # metadata (the varlen max_seqlen_k): with at most 1024 keys the library
    # skips the short-query launches, which would find no work
    max_kv = int(batch.kv_lengths.max()) if len(batch.kv_lengths) else 0

    def step():
        jfa.forward(q, k, v, qo, ko, bias, wl.causal, out=out, lse=lse, max_kv_len=max_kv)
        jfa.backward(q, k, v, out, lse, do, qo, ko, bias, wl.causal, dq=dq, dk=dk, dv=dv, bias_grad=bias_grad,
                     max_kv_len=max_kv)

    pw = prewarm(step, torch, prewarm_ms) if prewarm_ms > 0 else (0, 0.0)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-kernel durations: the same steps again, with the library's HIP
    # events recorded on the launch stream around every kernel (kept out of
    # the wall-clock pass above, whose launches they would space out).
    jfa.timing_collect()  # drop anything recorded before
    jfa.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    jfa.timing_enable(False)
    kt = jfa.timing_collect()

    cold = cold_cache_steps(step, cold_steps, torch) if cold_steps > 0 else None
    pairs = valid_pairs(batch.q_lengths, batch.kv_lengths, wl.causal)
    fwd_flops = 4.0 * wl.D * wl.H * pairs
    bwd_flops = 10.0 * wl.D * wl.H * pairs
    ms_step = (t1 - t0) * 1e3 / steps
    per = {k_: (ms / max(n, 1), n) for k_, (ms, n) in kt.items()}
    # forward: work lists, short-query chunks, forward; backward: work lists
    # with Delta, short-query chunks, dK/dV, dQ (and the bias-gradient sums)
    fwd_ms = (kt["plan"][0] + kt["forward"][0] + kt["fsq"][0]) / steps
    bwd_ms = (kt["bwd_prep"][0] + kt["dkdv"][0] + kt["dq"][0] + kt["sq"][0] + kt["dbias"][0]) / steps
    res = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "D": wl.D, "dtype": wl.dtype, "causal": wl.causal,
        "bias": wl.bias, "seed": wl.seed if seed is None else seed, "total_q": batch.total_q,
        "total_kv": batch.total_kv, "max_kv_len": max_kv, "valid_pairs_per_head": pairs,
        "ms_per_step": ms_step, "prewarm": {"steps": pw[0], "ms": pw[1]},
        "tflops_step": (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12,
        "fwd_ms_kernels": fwd_ms, "bwd_ms_kernels": bwd_ms,
        "fwd_tflops": fwd_flops / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
        "kernel_avg_ms": {k_: per[k_][0] for k_ in per if per[k_][1] > 0},
    }
    if cold is not None:
        res["cold_cache"] = {"steps": cold_steps, "flush_mib": 512, "median_ms": cold[0], "p10_ms": cold[1],
                             "p90_ms": cold[2], "tflops_median": (fwd_flops + bwd_flops) / (cold[0] * 1e-3) / 1e12}
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    res["fwd_pct_peak"] = 100.0 * res["fwd_tflops"] / peak
    res["bwd_pct_peak"] = 100.0 * res["bwd_tflops"] / peak
    # dominant kernel; its bound is the roofline its arithmetic intensity falls under
    share = {k_: kt[k_][0] for k_ in ("forward", "fsq", "dkdv", "dq", "sq")}
    dom = max(share, key=share.get)
    avg_ms = kt[dom][0] / kt[dom][1]
    kpairs = valid_pairs(batch.q_lengths, batch.kv_lengths, wl.causal, KERNEL_SEQS[dom])
    alg = KERNEL_FLOPS_PER_PAIR_D[dom] * wl.D * wl.H * kpairs
    executed = KERNEL_EXEC_FLOPS_PER_PAIR_D[dom] * wl.D * wl.H * kpairs
    alg_bytes = algorithmic_bytes(dom, batch)
    label = f"jfa_{'fwd' if dom == 'forward' else dom}_kernel<{wl.dtype},D={wl.D}{',bias' if wl.bias else ''}>"
    hbm = executed / max(alg_bytes, 1) < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm:
        achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "mfma_frac": alg / (avg_ms * 1e-3) / 1e12 / peak}
    else:
        achieved = alg / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    res["roofline"] = {"kernel": label, **roof, "traffic": recorded_traffic(label, idx), "traffic_unit": "bytes/launch",
                       "avg_launch_ms": avg_ms, "algorithmic_flops_per_launch": alg,
                       "executed_flops_per_launch": executed, "algorithmic_bytes_per_launch": alg_bytes}
    if padded_steps > 0 and wl.dtype == "bf16":  # the padded-dense kernels are bf16 only
        res["padded_baseline"] = run_padded(batch, d=dict(q=q, k=k, v=v, do=do, bias=bias, out=out, lse=lse, dq=dq),
                                            steps=padded_steps, jfa_ms=ms_step, jfa_fwd_ms=fwd_ms, jfa_bwd_ms=bwd_ms,
                                            torch=torch, jfa=jfa)
    res["_batch"] = batch
    return res


def run_padded(batch, d, steps, jfa_ms, jfa_fwd_ms, jfa_bwd_ms, torch, jfa):
    """The padded-dense baseline on the same batch: every sequence copied into a
    zeroed slot of the longest sequence's length, forward with a -inf key mask
    on every block, backward over every block (jfa_fwd_padded /
    jfa_bwd_padded). Returns its step time, the speedup of the jagged path and
    the memory ratio; the slots' valid rows are checked against the jagged
    outputs."""
    from variable_length_attention_jfa_amd import padded
    wl = batch.wl
    qo, ko = batch.q_offsets, batch.kv_offsets
    q_slot, kv_slot = int(batch.q_lengths.max()), int(batch.kv_lengths.max())
    qp, dop = padded.to_slots(d["q"], qo, q_slot), padded.to_slots(d["do"], qo, q_slot)
    kp, vp = padded.to_slots(d["k"], ko, kv_slot), padded.to_slots(d["v"], ko, kv_slot)
    kv_lens = torch.from_numpy(batch.kv_lengths.astype(np.int32)).to(qp.device)
    outp, lsep = torch.empty_like(qp), torch.empty(qp.shape[:3], dtype=torch.float32, device=qp.device)
    dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)

    def step():
        jfa.forward_padded(qp, kp, vp, kv_lens, d["bias"], wl.causal, out=outp, lse=lsep)
        jfa.backward_padded(qp, kp, vp, outp, lsep, dop, kv_lens, d["bias"], wl.causal, dq=dqp, dk=dkp, dv=dvp)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    jfa.timing_collect()
    jfa.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    jfa.timing_enable(False)
    kt = jfa.timing_collect()
    fwd_ms = (kt["plan"][0] + kt["forward"][0]) / steps
    bwd_ms = (kt["bwd_prep"][0] + kt["dkdv"][0] + kt["dq"][0]) / steps
    # the same valid rows as the jagged path (different block order and masking: rounding-level differences)
    diff_o = float((padded.from_slots(outp, qo).float() - d["out"].float()).abs().max()) if batch.total_q else 0.0
    diff_dq = float((padded.from_slots(dqp, qo).float() - d["dq"].float()).abs().max()) if batch.total_q else 0.0
    B, H, D = len(batch.q_lengths), wl.H, wl.D
    elt = 2 if wl.dtype == "bf16" else 4
    slot_b = padded.slot_bytes(B, q_slot, kv_slot, H, D, elt)
    jag_b = padded.jagged_bytes(batch.total_q, batch.total_kv, H, D, elt)
    scores_b = B * H * q_slot * kv_slot * 4  # a materialised fp32 score matrix of dense attention
    del qp, dop, kp, vp, outp, lsep, dqp, dkp, dvp
    return {"q_slot": q_slot, "kv_slot": kv_slot, "ms_per_step": ms, "fwd_ms_kernels": fwd_ms,
            "bwd_ms_kernels": bwd_ms, "steps": steps,
            "speedup_step": ms / jfa_ms, "speedup_fwd": fwd_ms / jfa_fwd_ms, "speedup_bwd": bwd_ms / jfa_bwd_ms,
            "padded_bytes": slot_b, "jagged_bytes": jag_b, "memory_ratio": slot_b / jag_b,
            "dense_scores_bytes": scores_b, "dense_memory_ratio": (slot_b + scores_b) / jag_b,
            "max_abs_diff_out_vs_jagged": diff_o, "max_abs_diff_dq_vs_jagged": diff_dq}


def algorithmic_bytes(kernel: str, batch) -> int:
    """Bytes the kernel must move at least once over the sequences it handles:
    its inputs read, its outputs written."""
    wl = batch.wl
    e = 2 if wl.dtype == "bf16" else 4
    short = (batch.q_lengths <= SHORT_Q_MAX) & (batch.kv_lengths > SHORT_KV_MIN)
    sel = short if KERNEL_SEQS[kernel] == "short" else ~short
    nq, nk = int(batch.q_lengths[sel].sum()), int(batch.kv_lengths[sel].sum())
    tq, tk = nq * wl.H * wl.D * e, nk * wl.H * wl.D * e
    rows = nq * wl.H * 4
    if kernel in ("forward", "fsq"):  # q, k, v in; out, lse out
        return tq + 2 * tk + tq + rows
    if kernel == "dkdv":         # q, k, v, dout, lse, delta in; dk, dv out
        return 2 * tq + 2 * tk + 2 * rows + 2 * tk
    if kernel == "sq":           # q, k, v, dout, lse, delta in; dq, dk, dv out (whole sequences)
        return 3 * tq + 4 * tk + 2 * rows
    return 2 * tq + 2 * tk + 2 * rows + tq   # dq: q, k, v, dout, lse, delta in; dq out


def _cpu_worker(wl_idx, seed, pairs, barrier, results):
    """One process of the CPU baseline: regenerates the batch from its seed
    (the same bytes the GPU gets), waits for the other processes, then times
    the oracle's forward and backward on its share of the (b, h) slices."""
    import oracle
    from variable_length_attention_jfa_amd import inputs as gen
    wl = gen.WORKLOADS[wl_idx]
    batch = gen.make_batch(wl, seed=seed)
    args = (batch.q, batch.k, batch.v)
    barrier.wait()
    t0 = time.perf_counter()
    out, lse = oracle.forward(*args, batch.q_offsets, batch.kv_offsets, batch.bias, wl.causal, pairs=pairs)
    t1 = time.perf_counter()
    barrier.wait()
    t2 = time.perf_counter()
    oracle.backward(*args, batch.dout, batch.q_offsets, batch.kv_offsets, batch.bias, wl.causal, pairs=pairs,
                    out=out, lse=lse)
    t3 = time.perf_counter()
    results.put((t1 - t0, t3 - t2, len(pairs)))


def cpu_baseline(wl_idx, seed=None, budget_gflop=600.0, max_procs=16):
    """The fp64 oracle on the host cores: one process per core (at most
    max_procs, the host share of one GPU), one BLAS thread each, the (b, h)
    slices split longest-first over the processes. The sample is the whole
    workload if its forward + backward stays under budget_gflop, else
    slices in a fixed shuffled order up to that budget. The forward and the
    backward (given the forward's O and lse) are timed separately as the
    slowest process's time, all processes starting each phase together.
    Runs before the GPU is touched: the processes are started fresh
    (spawn), never forked from a process holding GPU state."""
    import multiprocessing as mp
    from variable_length_attention_jfa_amd import inputs as gen
    wl = gen.WORKLOADS[wl_idx]
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    ql = wl.q_len.sample(rng, wl.B)
    kl = wl.kv_len.sample(rng, wl.B) if wl.kv_len is not None else ql
    B, H = len(ql), wl.H
    order = [(b, h) for h in range(H) for b in range(B)]
    np.random.default_rng(0).shuffle(order)
    pair_gflop = {}
    chosen, total = [], 0.0
    for b, h in order:
        p = valid_pairs(np.array([ql[b]]), np.array([kl[b]]), wl.causal)
        f = 14.0 * wl.D * p / 1e9
        if chosen and total + f > budget_gflop:
            break
        chosen.append((b, h))
        pair_gflop[(b, h)] = f
        total += f
    cores = max(1, min(len(os.sched_getaffinity(0)), max_procs))
    nproc = min(cores, len(chosen))
    shares = [[] for _ in range(nproc)]
    load = [0.0] * nproc
    for bh in sorted(chosen, key=lambda x: -pair_gflop[x]):  # longest first onto the least-loaded process
        i = int(np.argmin(load))
        shares[i].append(bh)
        load[i] += pair_gflop[bh]
    saved = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        barrier, results = ctx.Barrier(nproc), ctx.Queue()
        procs = [ctx.Process(target=_cpu_worker, args=(wl_idx, seed, sh, barrier, results)) for sh in shares]
        for pr in procs:
            pr.start()
        got = [results.get(timeout=600) for _ in procs]
        for pr in procs:
            pr.join()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    t_fwd = max(g[0] for g in got)
    t_bwd = max(g[1] for g in got)
    pairs = sum(valid_pairs(np.array([ql[b]]), np.array([kl[b]]), wl.causal) for b, _ in chosen)
    fwd_f, bwd_f = 4.0 * wl.D * pairs, 10.0 * wl.D * pairs
    return {"value": (fwd_f + bwd_f) / (t_fwd + t_bwd) / 1e12, "unit": "TFLOPS", "cores": nproc, "kind": "oracle",
            "fwd_tflops": fwd_f / t_fwd / 1e12, "bwd_tflops": bwd_f / t_bwd / 1e12, "fwd_s": t_fwd, "bwd_s": t_bwd,
            "sample": f"fp64 numpy oracle, {nproc} processes x 1 BLAS thread, on {len(chosen)} of {B * H} (b, h) "
                      f"slices of the same workload ({'all of it' if len(chosen) == B * H else 'a shuffled subset'}; "
                      f"{(fwd_f + bwd_f) / 1e9:.1f} valid-pair GFLOP): forward {t_fwd:.2f} s, backward given "
                      f"the forward's O and lse {t_bwd:.2f} s (slowest process of each phase)"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps first (the clocks settle within about 50 ms)")
    ap.add_argument("--workload", type=int, default=2, help="workload number 1..5 (default 2)")
    ap.add_argument("--also", type=str, default="1,3,4,5", help="comma list of extra workloads reported alongside")
    ap.add_argument("--all", action="store_true", help="also report workloads 1..5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true", help="skip the padded-dense baseline")
    ap.add_argument("--lib", default=None, help="run another build of the library (study variants)")
    ap.add_argument("--cpu-budget", type=float, default=600.0,
                    help="GFLOP of oracle work (forward + backward) the CPU baseline's sample may hold")
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="wall time of untimed steps before the --warmup steps (clock ramp-up)")
    ap.add_argument("--bias-grad", action="store_true",
                    help="the backward also returns the bias-table gradient (workloads with a bias)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run a plain device copy of MB mebibytes (reference for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the library computes one GPU's share; sharding across GPUs is not implemented)",
              file=sys.stderr)
        return 2

    # The CPU baseline first, before anything touches the GPU: its worker
    # processes start from a clean interpreter.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, budget_gflop=args.cpu_budget)
        print(f"[bench] cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    import torch
    from variable_length_attention_jfa_amd import inputs as gen
    from variable_length_attention_jfa_amd import jfa
    if args.lib:
        jfa.LIB_PATH = os.path.abspath(args.lib)
    jfa.lib()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    if args.bias_grad and not gen.WORKLOADS[args.workload].bias:
        print(f"bench.py: workload {args.workload} has no bias; --bias-grad needs one", file=sys.stderr)
        return 2
    pad_steps = 0 if args.no_padded else max(3, min(20, args.steps // 10))
    main_res = run_workload(args.workload, args.steps, args.warmup, torch, jfa, gen, bias_grad=args.bias_grad,
                            padded_steps=pad_steps, cold_steps=max(5, min(50, args.steps // 6)),
                            prewarm_ms=args.prewarm_ms)
    pb = main_res.get("padded_baseline")
    print(f"[bench] workload {args.workload}: {main_res['tflops_step']:.1f} TFLOP/s fwd+bwd, "
          f"fwd {main_res['fwd_tflops']:.1f} bwd {main_res['bwd_tflops']:.1f}"
          + (f"; padded-dense {pb['ms_per_step']:.2f} ms/step, speedup {pb['speedup_step']:.2f}x, "
             f"memory {pb['memory_ratio']:.2f}x" if pb else ""), file=sys.stderr, flush=True)
    extra_ids = list(range(1, 6)) if args.all else [int(x) for x in args.also.split(",") if x.strip()]
    extras = []
    for i in extra_ids:
        if i == args.workload:
            continue
        r = run_workload(i, max(3, args.steps // 2), 2, torch, jfa, gen, padded_steps=pad_steps,
                         prewarm_ms=min(100.0, args.prewarm_ms))
        r.pop("_batch")
        pb = r.get("padded_baseline")
        rf = r["roofline"]
        print(f"[bench] workload {i}: fwd {r['fwd_tflops']:.1f} ({r['fwd_pct_peak']:.1f}%) "
              f"bwd {r['bwd_tflops']:.1f} ({r['bwd_pct_peak']:.1f}%); {rf['kernel']} {rf['achieved']:.1f} "
              f"{rf['unit']} ({100 * rf['frac']:.1f}% of {rf['bound']})"
              + (f"; padded-dense {pb['ms_per_step']:.2f} ms/step, speedup {pb['speedup_step']:.2f}x, "
                 f"memory {pb['memory_ratio']:.2f}x" if pb else ""), file=sys.stderr, flush=True)
        extras.append(r)
        torch.cuda.empty_cache()

    batch = main_res.pop("_batch")

    wl = batch.wl
    line = {
        "metric": "jagged attn fwd/bwd TFLOPS (valid tokens) bf16 + % MFMA peak, 1 MI355X",
        "value": main_res["tflops_step"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "prewarm": main_res["prewarm"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B}, lengths U[{wl.q_len.lo},{wl.q_len.hi}], H={wl.H}, "
                               f"D={wl.D}, {wl.dtype}, causal={wl.causal}, bias={wl.bias}",
                   "B": wl.B, "H": wl.H, "D": wl.D, "bias_grad": args.bias_grad, "seed": main_res["seed"],
                   "total_tokens": main_res["total_q"], "max_kv_len": main_res["max_kv_len"],
                   "valid_pairs_per_head": main_res["valid_pairs_per_head"]},
        "pct_mfma_peak": 100.0 * main_res["tflops_step"] / PEAK_BF16_TFLOPS,
        "fwd_tflops": main_res["fwd_tflops"], "fwd_pct_peak": main_res["fwd_pct_peak"],
        "bwd_tflops": main_res["bwd_tflops"], "bwd_pct_peak": main_res["bwd_pct_peak"],
        "kernel_avg_ms": main_res["kernel_avg_ms"],
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "padded_baseline": main_res.get("padded_baseline"),
        "cold_cache": main_res.get("cold_cache"),
        "other_workloads": extras,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
