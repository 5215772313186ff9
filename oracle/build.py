"""Build the C oracle (test infrastructure) with gcc: oracle/libkvc_oracle.so."""
from __future__ import annotations

import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "kvc_oracle.c"
OUT = HERE / "libkvc_oracle.so"

# -ffp-contract=off: no fused multiply-add, so the fp64 arithmetic is exactly
# the operation order written in the source.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build() -> pathlib.Path:
    tmp = OUT.with_suffix(".so.tmp")
    cmd = ["gcc", *CFLAGS, "-o", str(tmp), str(SRC), "-lm"]
    subprocess.run(cmd, check=True)
    tmp.replace(OUT)
    return OUT


if __name__ == "__main__":
    print(build(), file=sys.stderr)
