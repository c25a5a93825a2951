"""Compile the fp64 oracle (plain C, gcc + OpenMP) into oracle/libsaga_oracle.so.

Test infrastructure: building the checker is not using it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "saga_oracle.c")
OUT = os.path.join(HERE, "libsaga_oracle.so")


def build(src: str = SRC, out: str = OUT, extra: list[str] | None = None) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           src, "-o", out + ".tmp", "-lm"] + list(extra or [])
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
