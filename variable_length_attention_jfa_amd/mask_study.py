"""Instruction-mix study of the forward's jagged edges: the method's
subtraction of the pad terms ("Jagged Flash Attention (JFA)", section "Four
generations", item 1) against -inf masking, on the same kernel.

Mode 0 is the library as built. Modes 1 and 2 are the same sources compiled
with JFA_FWD_MASK_MODE: 1 masks keys past a sequence's end with -inf in the
block that holds them, 2 bounds-checks every key of every block, as a kernel
over padded tensors would.

    python -m variable_length_attention_jfa_amd.mask_study --build
    python -m variable_length_attention_jfa_amd.mask_study --mode M --workload W
    rocprofv3 --pmc <counters> -- python -m variable_length_attention_jfa_amd.mask_study --mode M --workload W

A run times `--steps` forward calls with the library's HIP events and prints
one JSON line; under rocprofv3 the counters of the same launches are
collected. Every mode's output is checked against mode 0's on the same
inputs first.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
MODES = {0: "subtract pad terms (the method)", 1: "-inf mask on the block holding pad keys",
         2: "-inf bounds check on every block"}


def lib_path(mode: int) -> str:
    if mode == 0:
        return os.path.join(PKG, "libjfa.so")
    return os.path.join(PKG, "_study", f"libjfa_mask{mode}.so")


def build_variants(jobs: int = 8) -> None:
    from . import build as b
    for mode in (1, 2):
        b.build(jobs=jobs, defines=[f"JFA_FWD_MASK_MODE={mode}"], out=lib_path(mode),
                objdir=os.path.join(b.BUILD, f"mask{mode}"))


def _load(jfa, mode: int) -> None:
    path = lib_path(mode)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m variable_length_attention_jfa_amd.mask_study --build)")
    jfa._LIB = None
    jfa.LIB_PATH = path
    jfa.lib()


def run(mode: int, workload: int, steps: int, warmup: int) -> dict:
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

    _load(jfa, 0)
    ref_o, ref_l = jfa.forward(q, k, v, qo, ko, bias, wl.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = ref_o.float().cpu(), ref_l.cpu()
    if mode != 0:
        _load(jfa, mode)
    for _ in range(warmup):
        jfa.forward(q, k, v, qo, ko, bias, wl.causal)
    torch.cuda.synchronize()
    jfa.timing_collect()
    jfa.timing_enable(True)
    for _ in range(steps):
        out, lse = jfa.forward(q, k, v, qo, ko, bias, wl.causal)
    torch.cuda.synchronize()
    jfa.timing_enable(False)
    kt = jfa.timing_collect()
    d_o = float((out.float().cpu() - ref_o).abs().max())
    d_l = float((lse.cpu() - ref_l).abs().max())
    ms, n = kt["forward"]
    return {"mode": mode, "masking": MODES[mode], "workload": wl.name, "D": wl.D, "dtype": wl.dtype,
            "causal": wl.causal, "bias": wl.bias, "fwd_kernel_ms": ms / max(n, 1), "launches": n,
            "max_abs_out_vs_mode0": d_o, "max_abs_lse_vs_mode0": d_l}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--build", action="store_true", help="compile the mode 1 and 2 libraries")
    ap.add_argument("--mode", type=int, choices=sorted(MODES), default=0)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    args = ap.parse_args(argv)
    if args.build:
        build_variants()
        return 0
    res = run(args.mode, args.workload, args.steps, args.warmup)
    print(json.dumps(res), flush=True)
    # the masking changes rounding order only (same exact softmax)
    return 0 if res["max_abs_out_vs_mode0"] < 2e-2 and res["max_abs_lse_vs_mode0"] < 1e-3 else 1


if __name__ == "__main__":
    sys.exit(main())
