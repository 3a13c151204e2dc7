"""Build libmla.so in-tree with hipcc for gfx950.

``build()`` always recompiles; ``ensure_built()`` builds only when the shared
library is missing.  The library is a plain C-ABI shared object (no torch
types), loaded by the ctypes binding in this package.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmla.so")
SOURCES = [os.path.join(CSRC, "mla_api.cpp"), os.path.join(CSRC, "mla_kernels.hip"),
           os.path.join(CSRC, "mla_merge.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def compile_command(out: str = LIB_PATH) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        f"-I{INCLUDE}", f"-I{CSRC}",
        # packed fp32 VALU ops stay disabled in every HIP translation unit
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument", "-Wl,--no-undefined",
        *SOURCES, "-o", out,
    ]


def build(verbose: bool = True) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print("[libmla] " + " ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=PKG_DIR, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("libmla build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def ensure_built() -> str:
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    build()
