"""Build the gfx950 HIP library ``libswiglu_mlp.so`` in-tree with hipcc.

Usage: ``python -m bwd_gemm_epilogue_amd.build`` (or ``build()`` from
Python).  Always recompiles.  Extra hipcc flags may be appended with the
environment variable ``SWIGLU_HIPCC_FLAGS`` (diagnostics only).
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libswiglu_mlp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # identical fp32 rounding in every kernel that computes h: no implicit
    # contraction of a*b+c into fma (explicit fmaf only)
    "-ffp-contract=off",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    src = os.path.join(CSRC, "swiglu_mlp.hip")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", tmp]
    cmd += shlex.split(os.environ.get("SWIGLU_HIPCC_FLAGS", ""))
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the packed-fp32 target feature; that note is harmless
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
