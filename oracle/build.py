"""Build the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure only; building the checker is not using it.
Flags: -O2, no fast-math, no FMA contraction, IEEE denormals (gcc default).
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(_HERE, "qgemm_oracle.c")]
OUT = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-pthread", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", *CFLAGS, *SOURCES, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
