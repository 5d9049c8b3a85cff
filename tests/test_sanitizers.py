"""Sanitizer runs, on the CPU only.

* The oracle (oracle.c) built with AddressSanitizer and
  UndefinedBehaviorSanitizer (every finding fatal) under the whole pin suite
  of tests/test_oracle_pins.py.
* The library's host code (argument checks, launch-shape and precision
  choice, batch planning: the host side of every translation unit, built
  with the sanitizers for the host compilation only, -Xarch_host) under the
  ABI tests of tests/test_abi.py.  Those calls return before any launch, so
  no GPU is needed; the device code is built as usual and never runs here.

Each run is a fresh interpreter with the ASan runtime preloaded (leak
detection off: the interpreter itself keeps allocations until exit).
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _env(asan=None):
    if asan is None:  # gcc's runtime, for the gcc-built oracle
        asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    return dict(os.environ, LD_PRELOAD=asan,
                ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
                    *SAN, "-fPIC", "-shared", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    env = dict(_env(), RLCA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from linear_recurrence_scan_row_amd import build

    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    out = str(tmp_path / "librlca_san.so")
    # the host compiler's (clang's) runtime, linked as a shared library; no
    # sanitizer for the device code
    build.build(extra=host_san, out=out,
                link_extra=["-Xarch_host", "-fsanitize=address,undefined",
                            "-Xarch_host", "-shared-libsan"])
    clang_rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert clang_rt, "clang's ASan runtime is missing"
    script = ("import sys; sys.path.insert(0, sys.argv[1]);"
              "from linear_recurrence_scan_row_amd import rlca; rlca.LIB_PATH = sys.argv[2];"
              "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
              "'-m', 'not gpu', 'tests/test_abi.py']))")
    r = subprocess.run([sys.executable, "-c", script, ROOT, out], cwd=ROOT,
                       env=_env(clang_rt[0]),
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
