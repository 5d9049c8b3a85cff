"""The library's gfx950 kernels, as built here, need no scratch memory: none
has a private segment or spills VGPRs to memory.  A kernel with memory spills
runs slower and makes the runtime provide scratch memory for its launches,
which allocation-free callers (rlca_gae_stats_noalloc) cannot count on.

The device code objects come from the build's own object files
(_build/librlca/*.o, written by build()): the offload bundle in each
object's .hip_fatbin section is unpacked with clang-offload-bundler and its
kernel descriptors read with llvm-readelf --notes.  CPU only."""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJS = sorted(glob.glob(os.path.join(ROOT, "_build", "librlca", "*.hip.o")))
LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]


def _kernels(obj, tmp):
    bundle = os.path.join(tmp, os.path.basename(obj) + ".bundle")
    code = os.path.join(tmp, os.path.basename(obj) + ".co")
    subprocess.run([TOOLS[0], "--dump-section", f".hip_fatbin={bundle}", obj,
                    os.path.join(tmp, "host.o")], check=True, capture_output=True)
    subprocess.run([TOOLS[1], "--unbundle", "--type=o",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={bundle}",
                    f"--output={code}"], check=True, capture_output=True)
    notes = subprocess.run([TOOLS[2], "--notes", code], check=True, capture_output=True,
                           text=True).stdout
    kernels, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            kernels.setdefault(cur, {})
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_spill_count):\s+(\d+)", line)
        if m and cur is not None:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not OBJS, reason="the library's objects are not built")
@pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools missing")
def test_no_kernel_needs_scratch_memory(tmp_path):
    total = 0
    offenders = []
    for obj in OBJS:
        ks = _kernels(obj, str(tmp_path))
        # descriptors of kernels only (device functions carry no private
        # segment entry of their own)
        ks = {k: v for k, v in ks.items() if "private_segment_fixed_size" in v}
        assert ks, f"no kernel descriptors read from {obj}"
        total += len(ks)
        offenders += [(os.path.basename(obj), k, v) for k, v in ks.items()
                      if v["private_segment_fixed_size"] != 0 or v.get("vgpr_spill_count", 0)]
    assert total > 500, total
    assert not offenders, offenders[:5]
