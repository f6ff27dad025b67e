"""Builds libjfa.so (gfx950) from csrc/ with hipcc, in place.

    python -m variable_length_attention_jfa_amd.build [--jobs N] [--save-temps] [--define N=V --out PATH]

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
    if verbose:
        print(f"built {out}")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="extra preprocessor definition (study variants, e.g. JFA_LDS_SWIZZLE=0)")
    ap.add_argument("--out", default=LIB, help="library path (default: the package's libjfa.so)")
    args = ap.parse_args(argv)
    out = os.path.abspath(args.out)
    objdir = BUILD if out == LIB else os.path.join(BUILD, os.path.splitext(os.path.basename(out))[0])
    build(args.jobs, args.save_temps, defines=args.define, out=out, objdir=objdir)
    return 0


if __name__ == "__main__":
    sys.exit(main())
