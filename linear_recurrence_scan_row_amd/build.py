"""Build the HIP library librlca.so for gfx950 (in-tree, next to this file).

Each csrc/*.hip translation unit (one per estimator plus the C-ABI host code)
is compiled in parallel to an object under _build/, then linked into one
shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "librlca.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Werror",
    "-Wno-unused-command-line-argument",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # let the hardware preload the leading kernel arguments into SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=None, out: str = LIB_PATH, jobs: int = 8,
          link_extra=None) -> str:
    """Compile every translation unit (up to `jobs` at once, with `extra`
    flags) and link `out` (with `link_extra` flags)."""
    tag = os.path.splitext(os.path.basename(out))[0]
    obj_dir = os.path.join(BUILD_DIR, tag)
    os.makedirs(obj_dir, exist_ok=True)
    pending = []
    objs = []
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *(extra or []), "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        pending.append((cmd, src))
    running = []
    failed = []
    while pending or running:
        while pending and len(running) < jobs:
            cmd, src = pending.pop(0)
            running.append((subprocess.Popen(cmd), src))
        proc, src = running.pop(0)
        if proc.wait() != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(failed)}")
    tmp = out + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(link_extra or []), "-o", tmp,
            *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


def build_floor(verbose: bool = False) -> str:
    """Compile the benchmark's streaming-floor kernel (bench_floor.hip beside
    bench.py, a measurement aid, not part of the library) into bench_floor.so."""
    src = os.path.join(ROOT, "bench_floor.hip")
    out = os.path.join(ROOT, "bench_floor.so")
    tmp = out + ".tmp"
    flags = [f for i, f in enumerate(FLAGS) if f != "-I" and (i == 0 or FLAGS[i - 1] != "-I")]
    cmd = [HIPCC, *flags, "-shared", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(verbose=True, extra=extra))
