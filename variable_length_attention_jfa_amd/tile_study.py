"""Tile-shape and schedule study of the forward kernel ("TLX-Optimized Jagged
Flash Attention", sections "Architecture Migration Is Not Just a Recompile"
and "Targeting FA4 Means Targeting the Highest Bar": tile shapes, how the
K/V ring is filled, and keeping the matrix unit fed while the softmax runs).

Variant "lib" is the library as built: 4 waves x 32 query rows per item,
64-key blocks, K/V staged through registers into a two-stage LDS ring, and
for rows of 256 bytes (bf16 D = 128) the LDS operands of two matrix products
read ahead. The others are the same sources compiled with other choices:

    n128     128-key blocks for rows of 128 bytes (bf16 D = 64)
    n32      32-key blocks for rows of 128 bytes: fewer registers, 4 waves per SIMD
    r64      64 query rows per wave (two halves sharing every K and V fragment),
             256 rows per item, for bf16 D <= 64
    b3       launch bound of 3 workgroups per CU for bf16 D = 64 rows
    pf0      D = 128 operand reads in the compiler's order (no read-ahead)
    wdma     D = 128 K/V ring filled by direct loads into LDS
    w32b3    D = 128 with 32-key blocks, direct loads and 3 workgroups per CU
             (3 waves per SIMD)
    pp       D = 128 two-group kernel: 8 waves, 256 rows per item, the two
             waves of each SIMD in opposite matrix / softmax phases
    pp64     the two-group kernel for D = 64 as well
    m16      bf16 D <= 64 with 16x16x32 matrix products (two 16-row query
             tiles per wave) in place of 32x32x16

    python -m variable_length_attention_jfa_amd.tile_study --build
    python -m variable_length_attention_jfa_amd.tile_study --variant V --workload W
    rocprofv3 --pmc <counters> -- python -m variable_length_attention_jfa_amd.tile_study --variant V --workload W

A run times `--steps` forward calls with the library's HIP events and prints
one JSON line with the largest difference from the library's output (the
variants sum in other orders, so they are compared with the oracle by the
GPU tests, not bit for bit).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
VARIANTS = {
    "lib": ("library: 4 waves, 64-key blocks, register-staged ring, D=128 read-ahead 2", ()),
    "n128": ("128-key blocks (bf16 D = 64)", ("JFA_FWD_BN=128",)),
    "n32": ("32-key blocks (bf16 D = 64): 127 VGPRs, 4 waves per SIMD", ("JFA_FWD_BN=32",)),
    "r64": ("64 query rows per wave, 256 per item (bf16 D <= 64)", ("JFA_FWD_ROWS_PER_WAVE=64",)),
    "b3": ("3 workgroups per CU bound (bf16 D = 64)", ("JFA_FWD_BLOCKS=3",)),
    "pf0": ("D = 128 operand reads in compiler order", ("JFA_FWD_PREFETCH=0",)),
    "wdma": ("D = 128 ring by direct loads to LDS", ("JFA_FWD_WIDE_DMA=1",)),
    "w32b3": ("D = 128: 32-key blocks, direct loads, 3 waves per SIMD",
              ("JFA_FWD_WIDE_BN=32", "JFA_FWD_WIDE_DMA=1", "JFA_FWD_WIDE_BLOCKS=3")),
    "pp": ("D = 128 two-group kernel (8 waves, 256 rows)", ("JFA_FWD_PINGPONG=1",)),
    "pp64": ("two-group kernel for D = 64 and 128", ("JFA_FWD_PINGPONG=1", "JFA_FWD_PINGPONG_NARROW=1")),
    "m16": ("16x16x32 matrix products (bf16 D <= 64)", ("JFA_FWD_MFMA16=1",)),
}


def lib_path(variant: str) -> str:
    if variant == "lib":
        return os.path.join(PKG, "libjfa.so")
    return os.path.join(PKG, "_study", f"libjfa_tile_{variant}.so")


def build_variants(jobs: int = 8) -> None:
    from . import build as b
    for v, (_, defines) in VARIANTS.items():
        if v != "lib":
            b.build(jobs=jobs, defines=list(defines), out=lib_path(v), objdir=os.path.join(b.BUILD, f"tile_{v}"))


def _load(jfa, variant: str) -> None:
    path = lib_path(variant)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m variable_length_attention_jfa_amd.tile_study --build)")
    jfa._LIB = None
    jfa.LIB_PATH = path
    jfa.lib()


def run(variant: str, workload: int, steps: int, warmup: int) -> dict:
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

    _load(jfa, "lib")
    ref_o, ref_l = jfa.forward(q, k, v, qo, ko, bias, wl.causal, max_kv_len=max_kv)
    torch.cuda.synchronize()
    ref_o, ref_l = ref_o.float().clone(), ref_l.clone()
    if variant != "lib":
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
    ms, n = kt["forward"]
    fin = torch.isfinite(ref_l)
    return {"variant": variant, "choice": VARIANTS[variant][0], "workload": wl.name, "D": wl.D,
            "causal": wl.causal, "fwd_kernel_ms": ms / max(n, 1), "launches": n,
            "max_abs_diff_out": float((out.float() - ref_o).abs().max()) if out.numel() else 0.0,
            "max_abs_diff_lse": float((lse[fin] - ref_l[fin]).abs().max()) if bool(fin.any()) else 0.0}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--build", action="store_true", help="compile the variant libraries")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default="lib")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    args = ap.parse_args(argv)
    if args.build:
        build_variants()
        return 0
    print(json.dumps(run(args.variant, args.workload, args.steps, args.warmup)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
