"""Build the oracle's shared library with the host C compiler (test infrastructure)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (plain C99, fp64, no fast-math, no FMA contraction)."""
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-Werror", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
