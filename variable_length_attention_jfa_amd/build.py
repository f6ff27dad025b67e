"""Builds libjfa.so (gfx950) from csrc/ with hipcc, in place.

    python -m variable_length_attention_jfa_amd.build [--jobs N] [--save-temps] [--define N=V --out PATH]
    python -m variable_length_attention_jfa_amd.build --studies   (the design-study variants, on demand)

Every source is compiled for gfx950 only, with packed fp32 VALU instructions
disabled, then linked into variable_length_attention_jfa_amd/libjfa.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjfa.so")
SOURCES = ["jfa_plan.hip", "jfa_fwd.hip", "jfa_fwd_sq.hip", "jfa_bwd.hip", "jfa_bwd_sq.hip", "jfa_api.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def source_hash() -> str:
    """Hash of the kernel and header sources a build compiles."""
    import hashlib
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h")):
                with open(os.path.join(d, name), "rb") as fh:
                    h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def is_current(path: str) -> bool:
    """A study variant at `path` exists and was built from the current sources
    (its .srchash stamp, written by build(), matches)."""
    stamp = path + ".srchash"
    if not (os.path.exists(path) and os.path.exists(stamp)):
        return False
    with open(stamp) as fh:
        return fh.read().strip() == source_hash()


def _compile(src: str, save_temps: bool, objdir: str = BUILD, defines=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd.insert(1, "--save-temps")
    r = subprocess.run(cmd, cwd=objdir, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    return obj


def build(jobs: int = 4, save_temps: bool = False, verbose: bool = True, defines=(), out: str = LIB,
          objdir: str = BUILD) -> str:
    """Compiles every source and links `out` (the library by default; other
    `defines` and paths build study variants next to it)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps, objdir, defines), SOURCES))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if out != LIB:  # study variants carry the hash of the sources they were built from
        with open(out + ".srchash", "w") as fh:
            fh.write(source_hash() + "\n")
    if verbose:
        print(f"built {out}")
    return out


def build_studies(jobs: int = 8) -> None:
    """The design-study variants (each a whole library with other compile-time
    choices, under _study/): -inf masking modes 1 and 2, the list-order and
    grid variants of the scheduling study, unswizzled LDS tiles, and the
    backward with dQ fused into the dK/dV pass (atomic adds, ordered
    partials), the paired dK/dV kernel for 128-byte rows, and the forward's
    tile-shape variants. Their GPU tests skip
    when they are not built."""
    from . import mask_study, sched_study, tile_study
    mask_study.build_variants(jobs)
    sched_study.build_variants(jobs)
    tile_study.build_variants(jobs)
    build(jobs=jobs, defines=["JFA_LDS_SWIZZLE=0"], out=os.path.join(PKG, "_study", "libjfa_noswz.so"),
          objdir=os.path.join(BUILD, "noswz"))
    for mode in (1, 2):  # dQ fused into the dK/dV pass: atomic adds, ordered partials
        build(jobs=jobs, defines=[f"JFA_BWD_DQ={mode}"], out=os.path.join(PKG, "_study", f"libjfa_bwddq{mode}.so"),
              objdir=os.path.join(BUILD, f"bwddq{mode}"))
    # the paired (two-role) dK/dV kernel for 128-byte rows as well
    build(jobs=jobs, defines=["JFA_DKV_ONE_ROLE_ROWB=64"], out=os.path.join(PKG, "_study", "libjfa_dkvpaired.so"),
          objdir=os.path.join(BUILD, "dkvpaired"))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="extra preprocessor definition (study variants, e.g. JFA_LDS_SWIZZLE=0)")
    ap.add_argument("--out", default=LIB, help="library path (default: the package's libjfa.so)")
    ap.add_argument("--studies", action="store_true", help="build the design-study variants instead")
    args = ap.parse_args(argv)
    if args.studies:
        build_studies(args.jobs)
        return 0
    out = os.path.abspath(args.out)
    objdir = BUILD if out == LIB else os.path.join(BUILD, os.path.splitext(os.path.basename(out))[0])
    build(args.jobs, args.save_temps, defines=args.define, out=out, objdir=objdir)
    return 0


if __name__ == "__main__":
    sys.exit(main())
