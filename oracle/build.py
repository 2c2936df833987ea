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


def build(verbose: bool = False, src: str = SRC, out: str = LIB_PATH,
          extra_flags=()) -> str:
    """Compiles `src` (the oracle, or a test's modified copy of it) into
    `out`; `extra_flags` go to gcc as they are (e.g. sanitizers)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
