"""Build the CPU oracle library (test infrastructure) with gcc.

Flags keep IEEE semantics: no fast-math, no FMA contraction, SSE arithmetic
(x86-64), so every FP32 operation in ``qrs_oracle.c`` is one correctly
rounded IEEE operation.
"""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "qrs_oracle.c")
OUT = os.path.join(_HERE, "libqrs_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fno-builtin-rintf",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build_oracle(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_oracle(verbose=True))
