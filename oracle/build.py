"""Build the CPU oracle (TEST INFRASTRUCTURE ONLY) with gcc.

-ffp-contract=off and no fast-math: each fp32 operation in the oracle must
be a single correctly rounded IEEE-754 step.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "pkv_oracle.c")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
