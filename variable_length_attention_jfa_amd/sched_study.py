"""Scheduling study of the forward: the longest-first work list and the
persistent workgroups ("Jagged Flash Attention (JFA)", sections "Why standard
FlashAttention falls short" and "Four generations", item 3) against a list in
sequence order and against one workgroup per work item, on the same kernel.

Variant 0 is the library as built. The others are the same sources compiled
with JFA_SCHED_LPT=0 (groups of the list in sequence order instead of longest
first) and/or JFA_SCHED_PERSISTENT=0 (a grid of one workgroup per list slot,
each taking one item, instead of compute units x resident workgroups taking
items until the list is empty).

    python -m variable_length_attention_jfa_amd.sched_study --build
    python -m variable_length_attention_jfa_amd.sched_study --variant V --workload W

A run times `--steps` forward calls with the library's HIP events and prints
one JSON line. Every item is computed by one workgroup whatever the order, so
each variant's output must equal variant 0's bit for bit; this is checked
first.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
VARIANTS = {
    0: ("longest-first list, persistent workgroups (the method)", ()),
    1: ("sequence-order list, persistent workgroups", ("JFA_SCHED_LPT=0",)),
    2: ("longest-first list, one workgroup per item", ("JFA_SCHED_PERSISTENT=0",)),
    3: ("sequence-order list, one workgroup per item", ("JFA_SCHED_LPT=0", "JFA_SCHED_PERSISTENT=0")),
}


def lib_path(variant: int) -> str:
    if variant == 0:
        return os.path.join(PKG, "libjfa.so")
    return os.path.join(PKG, "_study", f"libjfa_sched{variant}.so")


def build_variants(jobs: int = 8) -> None:
    from . import build as b
    for v, (_, defines) in VARIANTS.items():
        if v:
            b.build(jobs=jobs, defines=list(defines), out=lib_path(v), objdir=os.path.join(b.BUILD, f"sched{v}"))


def _load(jfa, variant: int) -> None:
    path = lib_path(variant)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m variable_length_attention_jfa_amd.sched_study --build)")
    jfa._LIB = None
    jfa.LIB_PATH = path
    jfa.lib()


def run(variant: int, workload: int, steps: int, warmup: int) -> dict:
    import numpy as np
    import torch
    from . import inputs as gen, jfa

    wl = gen.WORKLOADS[workload]
    batch = gen.make_batch(wl)
    dev = torch.device("cuda")
    if wl.dtype == "bf16":
        t = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = t(batch.q_bits), t(batch.k_bits), t(batch.v_bits)
    else:
        q, k, v = (torch.from_numpy(x).to(dev) for x in (batch.q, batch.k, batch.v))
    qo = torch.from_numpy(batch.q_offsets).to(dev)
    ko = torch.from_numpy(batch.kv_offsets).to(dev)
    bias = None if batch.bias is None else torch.from_numpy(batch.bias).to(dev)
    max_kv = int(batch.kv_lengths.max()) if len(batch.kv_lengths) else 0

    _load(jfa, 0)
    ref_o, ref_l = jfa.forward(q, k, v, qo, ko, bias, wl.causal, max_kv_len=max_kv)
    torch.cuda.synchronize()
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    if variant != 0:
        _load(jfa, variant)
    for _ in range(warmup):
        jfa.forward(q, k, v, qo, ko, bias, wl.causal, max_kv_len=max_kv)
    torch.cuda.synchronize()
    jfa.timing_collect()
    jfa.timing_enable(True)
    for _ in range(steps):
        out, lse = jfa.forward(q, k, v, qo, ko, bias, wl.causal, max_kv_len=max_kv)
    torch.cuda.synchronize()
    jfa.timing_enable(False)
    kt = jfa.timing_collect()
    same = bool(torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                            ref_o.view(torch.int16) if ref_o.dtype == torch.bfloat16 else ref_o)
                and torch.equal(lse, ref_l))
    ms, n = kt["forward"]
    return {"variant": variant, "scheduling": VARIANTS[variant][0], "workload": wl.name, "D": wl.D,
            "causal": wl.causal, "fwd_kernel_ms": ms / max(n, 1), "launches": n,
            "plan_ms": kt["plan"][0] / max(kt["plan"][1], 1), "bit_identical_to_variant0": same}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--build", action="store_true", help="compile the variant libraries")
    ap.add_argument("--variant", type=int, choices=sorted(VARIANTS), default=0)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    args = ap.parse_args(argv)
    if args.build:
        build_variants()
        return 0
    res = run(args.variant, args.workload, args.steps, args.warmup)
    print(json.dumps(res), flush=True)
    return 0 if res["bit_identical_to_variant0"] else 1


if __name__ == "__main__":
    sys.exit(main())
