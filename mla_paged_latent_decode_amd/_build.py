"""Build libmla.so in-tree with hipcc for gfx950.

``build()`` always recompiles; ``ensure_built()`` builds only when the shared
library is missing.  The library is a plain C-ABI shared object (no torch
types), loaded by the ctypes binding in this package.

The stage-1 kernel source is compiled once per group of template instances
(MLA_STAGE1_GROUP 0..9) and once for the rest (MLA_MAIN); the translation
units build in parallel and are linked into one library.  A second, separate
library, libmla_peaks.so, holds the measured-ceiling probes the benchmark runs
(`bench.py --peaks`); the decode path never loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmla.so")
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libmla_peaks.so")
PEAKS_SRC = os.path.join(CSRC, "mla_peaks.hip")
KERNELS = os.path.join(CSRC, "mla_kernels.hip")
# (source, extra defines) of every translation unit
UNITS = ([(os.path.join(CSRC, "mla_api.cpp"), []), (os.path.join(CSRC, "mla_merge.hip"), []),
          (os.path.join(CSRC, "mla_noalloc.hip"), []),
          (KERNELS, ["-DMLA_MAIN"])] +
         [(KERNELS, [f"-DMLA_STAGE1_GROUP={g}"]) for g in range(10)])
SOURCES = sorted({u[0] for u in UNITS} | {PEAKS_SRC})
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
            # packed fp32 VALU ops stay disabled in every HIP translation unit
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def compile_commands(obj_dir: str) -> list:
    cmds = []
    for i, (src, defs) in enumerate(UNITS):
        obj = os.path.join(obj_dir, f"unit{i}.o")
        cmds.append(([hipcc(), *_flags(), *defs, "-c", src, "-o", obj], obj))
    return cmds


def _run(cmd):
    res = subprocess.run(cmd, cwd=PKG_DIR, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln]
    return res.returncode, msgs


def build(verbose: bool = True) -> str:
    with tempfile.TemporaryDirectory(prefix="libmla_build_") as tmp:
        cmds = compile_commands(tmp)
        if verbose:
            for cmd, _ in cmds:
                print("[libmla] " + " ".join(cmd), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(_run, [c for c, _ in cmds]))
        msgs = [m for _, ms in results for m in ms]
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("libmla build failed:\n" + "\n".join(msgs))
        tmp_lib = LIB_PATH + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined",
                *[o for _, o in cmds], "-o", tmp_lib]
        if verbose:
            print("[libmla] " + " ".join(link), flush=True)
        rc, lmsgs = _run(link)
        if rc != 0:
            raise RuntimeError("libmla link failed:\n" + "\n".join(lmsgs))
        if verbose and (msgs or lmsgs):
            print("\n".join(msgs + lmsgs), file=sys.stderr)
        os.replace(tmp_lib, LIB_PATH)
        # the probe library: one translation unit, linked on its own
        tmp_peaks = PEAKS_LIB_PATH + ".tmp"
        cmd = [hipcc(), *_flags(), "-shared", PEAKS_SRC, "-o", tmp_peaks]
        if verbose:
            print("[libmla] " + " ".join(cmd), flush=True)
        rc, pmsgs = _run(cmd)
        if rc != 0:
            raise RuntimeError("libmla_peaks build failed:\n" + "\n".join(pmsgs))
        os.replace(tmp_peaks, PEAKS_LIB_PATH)
    return LIB_PATH


def ensure_built() -> str:
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH
