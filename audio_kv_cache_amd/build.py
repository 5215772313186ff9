"""Build libkvc.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m audio_kv_cache_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libkvc.so"
SOURCES = ["kvc_host.hip", "budget.hip", "score.hip", "sss_select.hip", "gather.hip",
           "voxzip.hip", "c3.hip", "wnw.hip",
           "check.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of the generated code on purpose.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", str(PKG.parent / "include"),
]


def _compile(src: str) -> pathlib.Path:
    obj = BUILD / (pathlib.Path(src).stem + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> pathlib.Path:
    BUILD.mkdir(exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp),
           *map(str, objs), "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    tmp.replace(LIB)
    if verbose:
        print(LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
