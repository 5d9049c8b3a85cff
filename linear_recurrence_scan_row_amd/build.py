"""Build the HIP library librlca.so for gfx950 (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "librlca.so")
SOURCES = [os.path.join(HERE, "csrc", "rlca.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Werror",
    "-Wno-unused-command-line-argument",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False, extra=None) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
