"""Compile the CPU oracle (plain C, gcc, no HIP) into oracle/liboracle_v41.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "v41_oracle.c")
LIB = os.path.join(HERE, "liboracle_v41.so")


def build(verbose: bool = False) -> str:
    # No fast-math and no FMA contraction: every double operation rounds once,
    # as written.
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
