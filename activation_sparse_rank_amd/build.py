"""Build libpi.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m activation_sparse_rank_amd.build [--jobs N]

Every source under csrc/ is compiled with hipcc for gfx950 only and linked
into ``activation_sparse_rank_amd/libpi.so``.  Objects go to ``_build/`` at
the repository root.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpi.so")

SOURCES = ["abi.hip", "k_predict.hip", "k_compact.hip", "k_gather.hip", "k_mfma.hip", "k_q4.hip", "k_place.hip", "k_stream.hip"]

ARCH = "gfx950"
CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # Packed fp32 VALU instructions stay off in every HIP object.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libpi.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
