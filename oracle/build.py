"""Build the CPU oracle library (plain C, gcc).  Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgso.so")
SOURCES = [os.path.join(HERE, "gso.c")]
DEPS = SOURCES + [os.path.join(HERE, "gso.h"), os.path.join(HERE, "gso_real.inc")]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in DEPS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-shared", "-fPIC", "-o", tmp] + SOURCES + ["-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
