"""Build libabsa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m sampled_block_sparse_amd.build [--verbose]
The library lands in sampled_block_sparse_amd/_lib/libabsa.so; objects go to
sampled_block_sparse_amd/_build/.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libabsa.so")

SOURCES = ["absa.cpp", "plan_kernels.hip", "attn_kernels.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -ffp-contract=off: no implicit FMA contraction; kernels call fma explicitly
# where they want one, and the sampler's fixed-point rule relies on plain
# IEEE products and quotients.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source additions. The attention kernels never see a NaN they must
# propagate (a NaN input gives an unspecified output), so fmax there needs no
# quieting of its operands: without this every max of MFMA accumulators is
# preceded by two canonicalising v_max ops and every max with -inf is kept.
EXTRA = {
    "attn_kernels.hip": ["-fno-honor-nans"],
}


def source_flags(src: str):
    """Compiler flags of one source file (COMMON plus its own additions)."""
    return [*COMMON, *EXTRA.get(src, [])]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    """Compile every source and link libabsa.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([cc, *source_flags(src), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
