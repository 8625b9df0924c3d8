"""Compile librlt.so (HIP for gfx950) in-tree.

    python -m cross_token_recurrent_amd.build        # or build() from __graft_entry__

Every source under csrc/ is compiled with hipcc for gfx950 into _build/, in parallel,
then linked into cross_token_recurrent_amd/librlt.so.  The persistent decoder's kernel
instances are compiled in four parts (one compiler process each).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librlt.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]
DEC_SMALL_PARTS = 4
# (source, object name, extra flags); the slowest units first
UNITS = [("dec_small.hip", f"dec_small_p{k}", [f"-DRLT_DEC_PART={k}"]) for k in range(DEC_SMALL_PARTS)] + [
    (src, os.path.splitext(src)[0], []) for src in
    ["dec_batched.hip", "api.cpp", "misc.hip", "gemm.hip", "wstream.hip", "enc_attn.hip", "score.hip", "sample.hip",
     "bptt.hip"]]


def _compile(unit) -> str:
    src, name, extra = unit
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(UNITS))) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
