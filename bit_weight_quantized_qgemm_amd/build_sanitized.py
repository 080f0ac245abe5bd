"""Builds a host-sanitized copy of the library for the CPU test tier.

Every source is compiled as in ``build.py``, with AddressSanitizer and
UndefinedBehaviorSanitizer applied to the host code only (each sanitizer flag
goes to the host compilation through ``-Xarch_host``; the gfx950 device code is
built unchanged). The result, ``_build_san/libqgemm_san.so``, is for CPU-only
runs of the host logic: argument validation, the planner and the blob-layout
sizes, which run without a GPU. Load it into a Python process with the ASan
runtime preloaded (``asan_runtime()``) and ``QGEMM_LIB`` pointing at it.

Usage: ``python -m bit_weight_quantized_qgemm_amd.build_sanitized``.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

from bit_weight_quantized_qgemm_amd import build as _b

BUILD = os.path.join(_b.HERE, "_build_san")
LIB = os.path.join(BUILD, "libqgemm_san.so")

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library links against."""
    r = subprocess.run([_b.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"clang ASan runtime not found: {r.stdout} {r.stderr}")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_b.hipcc()] + _b._flags() + HOST_SAN + ["-c", os.path.join(_b.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(_b.SOURCES))) as ex:
        objs = list(ex.map(_compile, _b.SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_b.hipcc(), f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-shared-libsan"] + HOST_SAN + \
        ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
