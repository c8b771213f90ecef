"""Build libbutler.so for gfx950 in-tree with hipcc.

    python query_aware_sparse_imp_amd/csrc/build.py [--jobs N]

Every .hip file in this directory is compiled to an object under ``_build/`` at the
repository root and linked into ``query_aware_sparse_imp_amd/libbutler.so``; the
bandwidth-measurement kernels in ``measure/`` go into a library of their own,
``query_aware_sparse_imp_amd/libbutler_measure.so``.  It always recompiles (a build is the
"does it compile" check).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libbutler.so")
OUT_MEASURE = os.path.join(PKG, "libbutler_measure.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("BUTLER_OFFLOAD_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    sub = os.path.basename(os.path.dirname(src))
    prefix = "" if os.path.dirname(src) == HERE else sub + "_"
    obj = os.path.join(BUILD, prefix + os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(HERE, "*.hip")))
    msrcs = sorted(glob.glob(os.path.join(HERE, "measure", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs + msrcs))
    _link(objs[:len(srcs)], OUT)
    _link(objs[len(srcs):], OUT_MEASURE)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources and {OUT_MEASURE} from {len(msrcs)}")
    return OUT


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
