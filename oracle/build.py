"""Compile the C oracle into ``oracle/liboracle.so`` with gcc (host only).

Plain IEEE arithmetic: -O2, no fast-math, no floating-point contraction, so
every multiply and add rounds exactly as written in ``oracle.c``.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build() -> str:
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
