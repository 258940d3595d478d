"""Build the HIP library ``libexl3.so`` in-tree for gfx950.

    python -m linear_exl3_input_amd.build      (or __graft_entry__.build())

Every source is compiled with hipcc for ``--offload-arch=gfx950`` and linked
into one shared library next to this file.  Packed-fp32 instructions are
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``) and fp
contraction is off, so the fp32 arithmetic is exactly the adds and multiplies
written in the kernels.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libexl3.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["exl3_host.cpp", "exl3_misc.hip", "exl3_moe.hip", "exl3_rulers.hip", "exl3_noalloc.hip", "gemm_dense.hip"] + [f"gemm_b{b}.hip" for b in range(1, 9)]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the EXL3 HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l
                    and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the library; always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
