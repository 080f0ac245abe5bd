"""Builds the gfx950 HIP library ``libqgemm.so`` in-tree with hipcc, and the
measurement probes ``libqgemm_probes.so`` beside it.

Usage: ``python -m bit_weight_quantized_qgemm_amd.build`` (or ``build()``).
Every source is compiled on each call; objects go to ``_build/`` next to this
file and the shared libraries beside it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")
PROBES_LIB = os.path.join(HERE, "libqgemm_probes.so")
PROBES_SOURCES = ["probes.hip"]
SOURCES = ["api.cpp", "repack.hip", "w4a16.hip", "w4a8.hip", "w2w4.hip", "wide.hip", "quant.hip", "w4g.hip", "sp24.hip",
           "bitplane_lo.hip", "bitplane_hi.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # packed fp32 VALU forms stay disabled on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBES_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
