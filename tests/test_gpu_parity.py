"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Sizes here let the oracle finish in seconds while still spanning several
tiles and a ragged tail; full-size workloads are in test_gpu_full.py.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import BF16_TOL, compare_backward, compare_forward, rel_l2, to_device, tol_for
from variable_length_attention_jfa_amd import inputs as gen
from variable_length_attention_jfa_amd import build, jfa

pytestmark = pytest.mark.gpu

# The design-study variants are whole libraries built on demand; a variant
# built from other sources than the library's would not compute the same
# thing, so those tests run only on a variant stamped with the current sources.
STUDY_SKIP = ("study variant not built from the current sources "
              "(python -m variable_length_attention_jfa_amd.build --studies)")


def _run(batch, with_bwd=True, max_kv_len=0):
    d = to_device(batch)
    out, lse = jfa.forward(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_offsets"], d["bias"], batch.wl.causal,
                           max_kv_len=max_kv_len)
    grads = None
    if with_bwd:
        grads = jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"],
                             batch.wl.causal, max_kv_len=max_kv_len)
    torch.cuda.synchronize()
    return out, lse, grads


def _check(batch, with_bwd=True, label="", max_kv_len=0):
    print(f"[case] {label} B={len(batch.q_lengths)} H={batch.wl.H} D={batch.wl.D} dtype={batch.wl.dtype} "
          f"causal={batch.wl.causal} bias={batch.wl.bias} Tq={batch.total_q} Tk={batch.total_kv} "
          f"max_kv_len={max_kv_len}", flush=True)
    tol = tol_for(batch)
    out, lse, grads = _run(batch, with_bwd, max_kv_len)
    e_o, e_l, _, _ = compare_forward(batch, out, lse)
    assert e_o <= tol["out"], f"forward error {e_o}"
    assert e_l <= tol["lse"], f"lse error {e_l}"
    if with_bwd:
        r = compare_backward(batch, *grads)
        assert max(r) <= tol["grad"], f"gradient errors {r}"


# Reduced copies of the five workloads: same H, D, dtype, mask and bias.
SMALL = {
    1: gen.WORKLOADS[1],
    2: gen.small_workload(gen.WORKLOADS[2], B=6, lo=1, hi=700, seed=21),
    3: gen.small_workload(gen.WORKLOADS[3], B=5, lo=1, hi=600, seed=31),
    4: gen.small_workload(gen.WORKLOADS[4], B=5, lo=1, hi=64, kv=(64, 900), seed=41),
    5: gen.small_workload(gen.WORKLOADS[5], B=3, lo=16, hi=1100, seed=51),
}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_workload_parity(cfg):
    _check(gen.make_batch(SMALL[cfg]), label=f"small cfg{cfg}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal,bias,asym", [(False, False, False), (True, False, False), (False, True, True),
                                              (True, False, True), (True, True, True)])
def test_feature_grid(dtype, D, causal, bias, asym):
    if dtype == "f32" and D == 128:
        batch = gen.make_batch(gen.Workload("grid", 2, 1, D, dtype, causal, bias, gen.LengthDist("uniform", 1, 30)))
        with pytest.raises(jfa.JFAError) as e:
            _run(batch)
        assert e.value.status == 3  # JFA_ERR_UNSUPPORTED
        return
    base = gen.Workload("grid", 4, 2, D, dtype, causal, bias, gen.LengthDist("uniform", 1, 300),
                        gen.LengthDist("uniform", 1, 330) if asym else None, seed=100 + D)
    _check(gen.make_batch(base), label=f"grid {dtype} D={D} causal={causal} bias={bias} asym={asym}")


@pytest.mark.parametrize("lengths", [
    ([0, 5, 0, 7], None),                     # empty query sequences
    ([3, 4, 2], [0, 6, 0]),                   # no keys for some sequences
    ([1, 1, 1], None),                        # single tokens
    ([63, 64, 65, 127, 128, 129], None),      # tile edges (64-key blocks, 128-row tiles)
    ([2048], None),                           # one long sequence
    ([200, 70], [5, 300]),                    # Lq > Lk and Lq < Lk
])
@pytest.mark.parametrize("causal,bias", [(False, False), (True, False), (False, True), (True, True)])
def test_edge_lengths(lengths, causal, bias):
    ql, kl = lengths
    wl = gen.Workload("edge", len(ql), 2, 64, "bf16", causal, bias, gen.LengthDist("fixed", 1, 1), seed=5)
    _check(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl), label=f"edge {ql} {kl} causal={causal} bias={bias}")


@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 64)])
@pytest.mark.parametrize("causal,bias", [(False, False), (True, False), (False, True), (True, True)])
def test_short_query_passes(dtype, D, causal, bias):
    """Sequences with at most 64 queries and more than 1024 keys take the
    key-split forward and the single-owner backward: key counts across
    several 1024-key chunks and ragged tiles, the 64/65 and 1024/1025
    boundaries in one batch with the query-tile forward and the split
    backward, and empty query or key sides."""
    ql = [64, 65, 1, 33, 0, 17, 40, 0, 5, 64]
    kl = [2500, 70, 1024, 1025, 300, 0, 131, 3000, 4097, 1024]
    wl = gen.Workload("sq", len(ql), 2, D, dtype, causal, bias, gen.LengthDist("fixed", 1, 1), seed=61)
    _check(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl), label=f"short-query {dtype} D={D} causal={causal} bias={bias}")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 32)])
@pytest.mark.parametrize("causal,bias", [(False, False), (True, True)])
def test_key_bound_broken_by_batch(dtype, D, causal, bias):
    """A key-count bound of at most 1024 that the batch breaks (keys up to
    4097) only switches the short-query passes off: every sequence then takes
    the query-tile and key-tile passes, which still match the oracle."""
    ql = [64, 65, 1, 33, 0, 17, 40, 0, 5, 64]
    kl = [2500, 70, 1024, 1025, 300, 0, 131, 3000, 4097, 1024]
    wl = gen.Workload("kb", len(ql), 2, D, dtype, causal, bias, gen.LengthDist("fixed", 1, 1), seed=62)
    _check(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl), label=f"broken key bound {dtype} D={D}", max_kv_len=1)


@pytest.mark.parametrize("cfg", [2, 3])
def test_key_bound_kept(cfg):
    """A true bound of at most 1024 keys: no short-query sequence exists, so
    the results are bit-identical to a call without the bound."""
    batch = gen.make_batch(SMALL[cfg])
    bound = int(batch.kv_lengths.max())
    assert bound <= 1024
    _check(batch, label=f"small cfg{cfg} with its key bound", max_kv_len=bound)
    a, b = _run(batch), _run(batch, max_kv_len=bound)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_single_head_d128_long_causal():
    wl = gen.Workload("h1", 2, 1, 128, "bf16", True, False, gen.LengthDist("fixed", 1, 1), seed=9)
    _check(gen.make_batch(wl, q_lengths=[1500, 3000]), label="H=1 long causal")


def test_many_short_sequences():
    wl = gen.Workload("many", 4096, 1, 64, "bf16", False, False, gen.LengthDist("uniform", 1, 8), seed=10)
    _check(gen.make_batch(wl), label="B=4096 short")


@pytest.mark.parametrize("causal", [False, True])
def test_largest_batch(causal):
    """B at its maximum (JFA_MAX_BATCH = 8192) with empty and short
    sequences: lists of 8192 groups per head, one item per sequence."""
    wl = gen.Workload("maxb", 8192, 2, 64, "bf16", causal, False, gen.LengthDist("uniform", 0, 6), seed=12 + causal)
    _check(gen.make_batch(wl), label=f"B=8192 causal={causal}")


def test_many_heads():
    """Hundreds of heads (B x H groups far above B) with ragged lengths and a bias table per head."""
    wl = gen.Workload("manyh", 12, 384, 64, "bf16", True, True, gen.LengthDist("uniform", 1, 70), seed=14)
    _check(gen.make_batch(wl), label="H=384")


def test_long_sequence_d64_noncausal():
    """One 8192-token sequence at D = 64 without a mask: 64 query tiles over
    128 key blocks each, next to a 3-token one (gradients compared whole and
    per (b, h))."""
    wl = gen.Workload("long64", 2, 1, 64, "bf16", False, False, gen.LengthDist("fixed", 1, 1), seed=15)
    _check(gen.make_batch(wl, q_lengths=[8192, 3], kv_lengths=[8192, 3]), label="L=8192 D=64")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_deterministic_bitwise(cfg):
    batch = gen.make_batch(SMALL[cfg])
    a = _run(batch)
    b = _run(batch)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_outputs_outside_sequences_untouched():
    """Canary rows after T in every output must keep their sentinel values."""
    batch = gen.make_batch(SMALL[3])
    d = to_device(batch)
    Tq, Tk, H, D = batch.total_q, batch.total_kv, batch.wl.H, batch.wl.D
    pad = 200
    out_buf = torch.full((Tq + pad, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.full((Tq + pad, H), 7.0, dtype=torch.float32, device="cuda")
    dq_buf = torch.full((Tq + pad, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    dk_buf = torch.full((Tk + pad, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    dv_buf = torch.full((Tk + pad, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    out, lse = jfa.forward(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_offsets"], None, True,
                           out=out_buf[:Tq], lse=lse_buf[:Tq])
    jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], None, True,
                 dq=dq_buf[:Tq], dk=dk_buf[:Tk], dv=dv_buf[:Tk])
    torch.cuda.synchronize()
    for t in (out_buf, lse_buf, dq_buf, dk_buf, dv_buf):
        assert torch.all(t[-pad:] == 7.0)
    e_o, e_l, _, _ = compare_forward(batch, out, lse)
    assert e_o <= BF16_TOL["out"] and e_l <= BF16_TOL["lse"]


@pytest.mark.parametrize("kernel", [jfa.KERNEL_FWD, jfa.KERNEL_BWD_DKDV, jfa.KERNEL_BWD_DQ, jfa.KERNEL_BWD_SQ,
                                    jfa.KERNEL_FWD_SQ])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_plan_bit_exact(kernel, causal, cfg):
    wl = gen.WORKLOADS[cfg]
    rng = np.random.default_rng(wl.seed)
    ql = wl.q_len.sample(rng, wl.B)
    kl = wl.kv_len.sample(rng, wl.B) if wl.kv_len is not None else ql
    qo, ko = gen.offsets_from_lengths(ql), gen.offsets_from_lengths(kl)
    _check_plan(qo, ko, wl.H, wl.D, causal, kernel)


_PLAN_KIND = {jfa.KERNEL_FWD: ("q", oracle.SHORT_Q_MAX), jfa.KERNEL_BWD_DKDV: ("kv", oracle.SHORT_Q_MAX),
              jfa.KERNEL_BWD_DQ: ("q", oracle.SHORT_Q_MAX), jfa.KERNEL_BWD_SQ: ("sq", None),
              jfa.KERNEL_FWD_SQ: ("sq", None)}


def _check_plan(qo, ko, H, D, causal, kernel):
    tm, tn = jfa.tile_config(kernel, D)
    kind, short_q = _PLAN_KIND[kernel]
    ref, starts, counts, first = oracle.build_plan_queues(qo, ko, H, tm, tn, causal, kind=kind, short_q=short_q,
                                                          n_queues=jfa.PLAN_QUEUES, with_groups=True)
    got = jfa.build_plan(torch.from_numpy(qo).cuda(), torch.from_numpy(ko).cuda(), H, D, causal, kernel,
                         int(qo[-1]), int(ko[-1]))
    hdr, items = got[0], got[1]
    torch.cuda.synchronize()
    if kernel in jfa.SQ_KERNELS:
        np.testing.assert_array_equal(got[2].cpu().numpy(), first)
    h = hdr.cpu().numpy()
    assert h[0] == len(ref) and h[1] == 0 and h[2] == jfa.PLAN_QUEUES
    np.testing.assert_array_equal(h[4:12], starts)
    np.testing.assert_array_equal(h[12:20], counts)
    np.testing.assert_array_equal(h[32:32 * 9:32], 0)  # tickets
    np.testing.assert_array_equal(items[:len(ref)].cpu().numpy(), ref)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 3000)) if seed else 8192
    ql = rng.integers(0, 3000, size=B) * (rng.random(B) < 0.9)
    kl = rng.integers(0, 5000, size=B) * (rng.random(B) < 0.9)
    qo, ko = gen.offsets_from_lengths(ql), gen.offsets_from_lengths(kl)
    H = int(rng.integers(1, 9))
    for kernel in (jfa.KERNEL_FWD, jfa.KERNEL_BWD_DKDV, jfa.KERNEL_BWD_DQ, jfa.KERNEL_BWD_SQ, jfa.KERNEL_FWD_SQ):
        for causal in (False, True):
            _check_plan(qo, ko, H, 128, causal, kernel)


@pytest.mark.parametrize("B", [0, 1, 5, 1023, 1024, 1025, 8192])
def test_offsets_bit_exact(B):
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 5000, size=B).astype(np.int32)
    got = jfa.offsets_from_lengths(torch.from_numpy(lens).cuda())
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.exclusive_scan(lens))


def test_invalid_arguments_raise():
    batch = gen.make_batch(SMALL[2])
    d = to_device(batch)
    L = jfa.lib()
    # D not supported
    st = L.jfa_fwd(jfa._ptr(d["q"]), jfa._ptr(d["k"]), jfa._ptr(d["v"]), jfa._ptr(d["q_offsets"]),
                   jfa._ptr(d["kv_offsets"]), 6, 8, 48, batch.total_q, batch.total_kv, 0, None, 0, jfa._ptr(d["q"]),
                   jfa._ptr(d["q"]), None, 0, None)
    assert st == 1
    # workspace too small
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    lse = torch.empty(batch.total_q, 8, dtype=torch.float32, device="cuda")
    need = L.jfa_fwd_workspace_bytes(6, 8, batch.total_q, batch.total_kv, 64, 0)
    st = L.jfa_fwd(jfa._ptr(d["q"]), jfa._ptr(d["k"]), jfa._ptr(d["v"]), jfa._ptr(d["q_offsets"]),
                   jfa._ptr(d["kv_offsets"]), 6, 8, 64, batch.total_q, batch.total_kv, 0, None, 0, jfa._ptr(out),
                   jfa._ptr(lse), jfa._ptr(ws), need - 16, None)
    assert st == 2
    assert b"workspace" in L.jfa_last_error()
    # misaligned q
    st = L.jfa_fwd(ctypes_offset(d["q"], 2), jfa._ptr(d["k"]), jfa._ptr(d["v"]), jfa._ptr(d["q_offsets"]),
                   jfa._ptr(d["kv_offsets"]), 6, 8, 64, batch.total_q, batch.total_kv, 0, None, 0, jfa._ptr(out),
                   jfa._ptr(lse), jfa._ptr(ws), 4096, None)
    assert st == 1
    # B = 0 is a no-op
    st = L.jfa_fwd(None, None, None, jfa._ptr(d["q_offsets"]), jfa._ptr(d["kv_offsets"]), 0, 8, 64, 0, 0, 0, None,
                   0, None, None, jfa._ptr(ws), 4096, None)
    assert st == 0


def ctypes_offset(t, nbytes):
    import ctypes
    return ctypes.c_void_p(t.data_ptr() + nbytes)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_masking_study_variants(mode, cfg):
    """The -inf masking variants of the instruction-mix study compute the same
    forward as the subtraction (the oracle decides)."""
    from variable_length_attention_jfa_amd import mask_study
    path = mask_study.lib_path(mode)
    if not build.is_current(path):
        pytest.skip(STUDY_SKIP)
    saved = jfa.LIB_PATH
    try:
        jfa._LIB = None
        jfa.LIB_PATH = path
        _check(gen.make_batch(SMALL[cfg]), with_bwd=False, label=f"masking mode {mode} cfg{cfg}")
    finally:
        jfa._LIB = None
        jfa.LIB_PATH = saved


_TILE_CASES = {
    # sizes spanning several tiles and ragged tails; causal, bias and
    # asymmetric lengths; every D the variants change
    "small_cfg2": lambda: gen.make_batch(SMALL[2]),
    "small_cfg3": lambda: gen.make_batch(SMALL[3]),
    "d128_causal_bias_asym": lambda: gen.make_batch(
        gen.Workload("tile", 6, 2, 128, "bf16", True, True, gen.LengthDist("fixed", 1, 1), seed=91),
        q_lengths=[300, 70, 1, 0, 257, 640], kv_lengths=[300, 40, 1, 5, 700, 640]),
    "d64_causal_bias_asym": lambda: gen.make_batch(
        gen.Workload("tile", 6, 2, 64, "bf16", True, True, gen.LengthDist("fixed", 1, 1), seed=92),
        q_lengths=[300, 70, 1, 0, 257, 640], kv_lengths=[300, 40, 1, 5, 700, 640]),
    "d32_causal_bias_asym": lambda: gen.make_batch(
        gen.Workload("tile", 6, 2, 32, "bf16", True, True, gen.LengthDist("fixed", 1, 1), seed=95),
        q_lengths=[300, 70, 1, 0, 257, 640], kv_lengths=[300, 40, 1, 5, 700, 640]),
    "edges_d64_causal": lambda: gen.make_batch(
        gen.Workload("tile", 8, 2, 64, "bf16", True, False, gen.LengthDist("fixed", 1, 1), seed=94),
        q_lengths=[31, 32, 33, 63, 64, 65, 255, 257], kv_lengths=[31, 32, 33, 63, 64, 65, 255, 257]),
    "edges_d128": lambda: gen.make_batch(
        gen.Workload("tile", 6, 2, 128, "bf16", False, False, gen.LengthDist("fixed", 1, 1), seed=93),
        q_lengths=[63, 64, 65, 255, 256, 257], kv_lengths=[63, 64, 65, 255, 256, 257]),
}


@pytest.mark.parametrize("variant", ["n128", "n32", "r64", "b3", "pf0", "wdma", "w32b3", "pp", "pp64", "m16"])
@pytest.mark.parametrize("case", sorted(_TILE_CASES))
def test_tile_study_variants(variant, case):
    """Every variant of the forward's tile-shape study computes the forward
    the oracle does (the study variants change tile shapes, the ring and the
    schedule, not the arithmetic of a row)."""
    from variable_length_attention_jfa_amd import tile_study
    path = tile_study.lib_path(variant)
    if not build.is_current(path):
        pytest.skip(STUDY_SKIP)
    saved = jfa.LIB_PATH
    try:
        jfa._LIB = None
        jfa.LIB_PATH = path
        _check(_TILE_CASES[case](), with_bwd=False, label=f"tile variant {variant} {case}")
    finally:
        jfa._LIB = None
        jfa.LIB_PATH = saved


def _check_dbias(batch, label, max_kv_len=0):
    print(f"[case] dbias {label} B={len(batch.q_lengths)} H={batch.wl.H} D={batch.wl.D} dtype={batch.wl.dtype} "
          f"causal={batch.wl.causal} Tq={batch.total_q} Tk={batch.total_kv} max_kv_len={max_kv_len}", flush=True)
    d = to_device(batch)
    args = (d["q"], d["k"], d["v"])
    out, lse = jfa.forward(*args, d["q_offsets"], d["kv_offsets"], d["bias"], batch.wl.causal, max_kv_len=max_kv_len)
    g0 = jfa.backward(*args, out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"], batch.wl.causal,
                      max_kv_len=max_kv_len)
    g1 = jfa.backward(*args, out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"], batch.wl.causal,
                      bias_grad=True, max_kv_len=max_kv_len)
    g2 = jfa.backward(*args, out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"], batch.wl.causal,
                      bias_grad=True, max_kv_len=max_kv_len)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(batch.q, batch.k, batch.v, batch.dout, batch.q_offsets, batch.kv_offsets, batch.bias,
                           batch.wl.causal)
    got = g1[3].cpu().numpy()
    e = rel_l2(got, ref)
    print(f"   dbias relL2={e:.3e} |ref|max={np.abs(ref).max():.3e} sum over bins={got.sum(axis=1)}", flush=True)
    assert e <= tol_for(batch)["grad"], f"bias gradient error {e}"
    assert torch.equal(g1[3], g2[3]), "bias gradient must be bit-identical run to run"
    for x, y in zip(g0, g1[:3]):  # asking for dbias leaves dq, dk, dv as they were
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_gradient(dtype, D, causal):
    """Bias gradient through the dK/dV pass (one-role and paired kernels) and
    the short-query owner: distances inside and beyond the clipping radius,
    several chunks, asymmetric and empty sequences."""
    ql = [300, 40, 0, 70, 5, 1, 600, 64]
    kl = [300, 2100, 500, 40, 1500, 1, 650, 1025]
    wl = gen.Workload("db", len(ql), 2, D, dtype, causal, True, gen.LengthDist("fixed", 1, 1), seed=71)
    _check_dbias(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl, with_dout=True), f"{dtype} D={D} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bias_gradient_key_bound_broken(causal):
    """The bias gradient with the short-query passes switched off by a bound
    the batch breaks: every sequence's bins come from the dK/dV pass."""
    ql = [300, 40, 0, 70, 5, 1, 600, 64]
    kl = [300, 2100, 500, 40, 1500, 1, 650, 1025]
    wl = gen.Workload("dbk", len(ql), 2, 64, "bf16", causal, True, gen.LengthDist("fixed", 1, 1), seed=73)
    _check_dbias(gen.make_batch(wl, q_lengths=ql, kv_lengths=kl, with_dout=True), f"broken key bound causal={causal}",
                 max_kv_len=1024)


def test_bias_gradient_workload4_small():
    _check_dbias(gen.make_batch(SMALL[4], with_dout=True), "small cfg4")


def test_bias_gradient_no_pairs():
    wl = gen.Workload("db0", 3, 2, 64, "bf16", False, True, gen.LengthDist("fixed", 1, 1), seed=72)
    batch = gen.make_batch(wl, q_lengths=[0, 0, 0], kv_lengths=[0, 0, 0], with_dout=True)
    d = to_device(batch)
    out = torch.empty_like(d["q"])
    lse = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    g = jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], d["bias"], False,
                     bias_grad=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g[3]) == 0


@pytest.mark.parametrize("variant", [1, 2, 3])
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_scheduling_study_variants(variant, cfg):
    """The list-order and grid variants of the scheduling study compute every
    work item the same way: their forward equals the library's bit for bit, and
    the oracle's within the tolerances."""
    from variable_length_attention_jfa_amd import sched_study
    path = sched_study.lib_path(variant)
    if not build.is_current(path):
        pytest.skip(STUDY_SKIP)
    batch = gen.make_batch(SMALL[cfg])
    ref = _run(batch, with_bwd=False)
    saved = jfa.LIB_PATH
    try:
        jfa._LIB = None
        jfa.LIB_PATH = path
        _check(batch, with_bwd=False, label=f"scheduling variant {variant} cfg{cfg}")
        got = _run(batch, with_bwd=False)
    finally:
        jfa._LIB = None
        jfa.LIB_PATH = saved
    assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)) and torch.equal(got[1], ref[1])


def test_binding_rejects_wrong_output_shapes():
    """Output buffers are written through plain pointers: the binding refuses
    any whose shape differs from what the call writes."""
    batch = gen.make_batch(SMALL[2])
    d = to_device(batch)
    args = (d["q"], d["k"], d["v"], d["q_offsets"], d["kv_offsets"], None, False)
    short = torch.empty((batch.total_q - 1,) + tuple(d["q"].shape[1:]), dtype=d["q"].dtype, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        jfa.forward(*args, out=short)
    out, lse = jfa.forward(*args)
    with pytest.raises(ValueError, match="shape"):
        jfa.backward(d["q"], d["k"], d["v"], out, lse, d["dout"], d["q_offsets"], d["kv_offsets"], None, False,
                     dk=d["k"][:-1])
    with pytest.raises(ValueError, match="shape"):
        jfa.backward(d["q"], d["k"], d["v"], out, lse[:-1], d["dout"], d["q_offsets"], d["kv_offsets"], None, False)
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bias", [False, True])
def test_subtraction_cancellation_guard(D, bias):
    """Every valid score ~20 below the pad keys' score (0, or the bias): in
    fp32 the pad terms absorb the valid ones, and subtracting them leaves
    nothing. The forward then sums the last block's valid terms again; O and
    lse must match the oracle, and the backward with them."""
    ql, kl = [4, 70, 9], [5, 70, 130]
    wl = gen.Workload("cancel", len(ql), 2, D, "bf16", False, bias, gen.LengthDist("fixed", 1, 1), seed=81)
    batch = gen.make_batch(wl, q_lengths=ql, kv_lengths=kl)
    a, b = 16.0, (10.0 if D == 64 else 14.0)  # score = -a * b / sqrt(D): -20 (D = 64), -19.8 (D = 128)
    for s in (0, 2):  # sequences 0 and 2: one block with 59 pad keys; two full blocks and 62 pads
        qs = slice(batch.q_offsets[s], batch.q_offsets[s + 1])
        ks = slice(batch.kv_offsets[s], batch.kv_offsets[s + 1])
        batch.q[qs] = 0.0
        batch.q[qs, :, 0] = a
        batch.k[ks, :, 0] = -b
    batch.q_bits = gen.bf16_round(batch.q)
    batch.k_bits = gen.bf16_round(batch.k)
    _check(batch, label=f"cancellation guard D={D} bias={bias}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bias", [False, True])
def test_subtraction_cancellation_guard_short_query(D, bias):
    """The same adversarial scores on the key-split forward of short-query
    sequences (at most 64 queries, more than 1024 keys): the chunk that holds
    the pad keys is the one that cancels."""
    ql, kl = [4, 9, 40], [1030, 2050, 1500]
    wl = gen.Workload("cancel_sq", len(ql), 2, D, "bf16", False, bias, gen.LengthDist("fixed", 1, 1), seed=82)
    batch = gen.make_batch(wl, q_lengths=ql, kv_lengths=kl)
    a, b = 16.0, (10.0 if D == 64 else 14.0)
    for s in (0, 1):
        qs = slice(batch.q_offsets[s], batch.q_offsets[s + 1])
        ks = slice(batch.kv_offsets[s], batch.kv_offsets[s + 1])
        batch.q[qs] = 0.0
        batch.q[qs, :, 0] = a
        batch.k[ks, :, 0] = -b
    batch.q_bits = gen.bf16_round(batch.q)
    batch.k_bits = gen.bf16_round(batch.k)
    _check(batch, label=f"short-query cancellation guard D={D} bias={bias}")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_unswizzled_lds_variant(cfg):
    """The bank-conflict study's build (LDS tiles stored unpermuted) reads what
    it writes in every kernel: forward and backward still match the oracle."""
    path = os.path.join(os.path.dirname(jfa.LIB_PATH), "_study", "libjfa_noswz.so")
    if not build.is_current(path):
        pytest.skip(STUDY_SKIP)
    saved = jfa.LIB_PATH
    try:
        jfa._LIB = None
        jfa.LIB_PATH = path
        _check(gen.make_batch(SMALL[cfg]), label=f"unswizzled LDS cfg{cfg}")
    finally:
        jfa._LIB = None
        jfa.LIB_PATH = saved


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_positive_bias_bin(D, causal):
    """One bias entry of 90 (exp(90) overflows fp32) at distance i - j = 40.
    Query rows past a sequence's end inside its last query block pair with
    valid keys at that distance; their P must be exactly 0 (their lse is set
    to +inf), or inf * 0 would carry NaN into every valid key's dK and dV of
    that block. Ragged last blocks of the dK/dV pass (one-role at D = 64,
    paired waves at D = 128) and a short-query sequence (40 queries, 1500
    keys) for the single-owner backward."""
    ql, kl = [70, 100, 33, 40, 129], [70, 100, 33, 1500, 129]
    wl = gen.Workload("bigbias", len(ql), 2, D, "bf16", causal, True, gen.LengthDist("fixed", 1, 1), seed=83)
    batch = gen.make_batch(wl, q_lengths=ql, kv_lengths=kl)
    batch.bias[:, 128 + 40] = 90.0  # bins are clip(i - j, -128, 128) + 128
    _check(batch, label=f"large bias bin D={D} causal={causal}")


_BWD_DQ_CASES = {
    "small_cfg2": lambda: gen.make_batch(SMALL[2]),
    "bf16_d32_causal_bias_asym": lambda: gen.make_batch(gen.Workload(
        "dqd", 4, 2, 32, "bf16", True, True, gen.LengthDist("uniform", 1, 300), gen.LengthDist("uniform", 1, 330),
        seed=131)),
    "bf16_d64_causal": lambda: gen.make_batch(gen.Workload(
        "dqd", 4, 2, 64, "bf16", True, False, gen.LengthDist("uniform", 1, 400), seed=132)),
    "f32_d32_bias_asym": lambda: gen.make_batch(gen.Workload(
        "dqd", 4, 2, 32, "f32", False, True, gen.LengthDist("uniform", 1, 200), gen.LengthDist("uniform", 1, 260),
        seed=133)),
    "edges": lambda: gen.make_batch(gen.Workload("dqd", 8, 2, 64, "bf16", False, False, gen.LengthDist("fixed", 1, 1),
                                                 seed=134),
                                    q_lengths=[0, 5, 1, 63, 64, 65, 128, 129], kv_lengths=[3, 0, 1, 63, 64, 65, 128, 129]),
    "short_query_mix": lambda: gen.make_batch(gen.Workload("dqd", 6, 2, 64, "bf16", False, True,
                                                           gen.LengthDist("fixed", 1, 1), seed=135),
                                              q_lengths=[64, 65, 1, 33, 17, 40], kv_lengths=[2500, 70, 1024, 1025, 0, 131]),
}


@pytest.mark.parametrize("case", sorted(_BWD_DQ_CASES))
@pytest.mark.parametrize("variant", ["bwddq1", "bwddq2", "dkvpaired"])
def test_backward_dq_design_variants(variant, case):
    """The backward-design study builds (dQ fused into the dK/dV pass: bwddq1
    with fp32 atomic adds, bwddq2 with per-key-tile partials summed in
    key-tile order; dkvpaired: the paired dK/dV kernel for 128-byte rows too)
    match the oracle like the library's passes."""
    path = os.path.join(os.path.dirname(jfa.LIB_PATH), "_study", f"libjfa_{variant}.so")
    if not build.is_current(path):
        pytest.skip(STUDY_SKIP)
    batch = _BWD_DQ_CASES[case]()
    saved = jfa.LIB_PATH
    try:
        jfa._LIB = None
        jfa.LIB_PATH = path
        _check(batch, label=f"backward design {variant} {case}")
    finally:
        jfa._LIB = None
        jfa.LIB_PATH = saved
