"""The benchmark's streaming-floor library (bench_floor.so, built by build()):
its launch description matches bench.py's, its multiply-high division by T
(the row-end test) is exact, and every benchmark workload's step, in every
storage type the benchmark runs it in, is a description the kernel takes.
No GPU call: bench_floor_prepare only checks and fills in the description."""
import ctypes
import os
import random

import numpy as np
import pytest
import torch

import bench
from linear_recurrence_scan_row_amd import workloads


@pytest.fixture(scope="module")
def floor():
    if not os.path.exists(bench.FLOOR_LIB):
        pytest.skip("bench_floor.so is not built")
    lib = ctypes.CDLL(bench.FLOOR_LIB)
    lib.bench_floor_launch_bytes.restype = ctypes.c_size_t
    lib.bench_floor_divide.restype = ctypes.c_uint32
    lib.bench_floor_divide.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    lib.bench_floor_prepare.restype = ctypes.c_int64
    lib.bench_floor_prepare.argtypes = [ctypes.POINTER(bench._FloorLaunch)]
    return lib


def test_layout_matches(floor):
    assert floor.bench_floor_launch_bytes() == ctypes.sizeof(bench._FloorLaunch)


def test_division_by_invariant_is_exact(floor):
    rng = random.Random(5)
    divisors = list(range(2, 3000)) + [rng.randrange(2, 1 << 32) for _ in range(3000)] + \
        [(1 << 31) - 1, 1 << 31, (1 << 32) - 1, 4096, 131072, 1 << 20]
    for d in divisors:
        for n in [0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, (1 << 31), (1 << 32) - 1] + \
                [rng.randrange(0, 1 << 32) for _ in range(20)]:
            n &= 0xFFFFFFFF
            assert floor.bench_floor_divide(n, d) == n // d, (n, d)
    assert floor.bench_floor_divide(7, 1) == 0xFFFFFFFF   # divisors below 2 are refused


def _buffers(arrays, real):
    """Stand-ins with each array's element size (floor_record reads only
    addresses and element sizes)."""
    bufs = {}
    for k, v in arrays.items():
        dt = real if v.dtype == np.float32 else torch.from_numpy(v[:1].copy()).dtype
        bufs[k] = torch.empty(1, dtype=dt)
    for k in ("o0", "o1"):
        bufs[k] = torch.empty(1, dtype=real)
    bufs["oi"] = torch.empty(1, dtype=torch.int32)
    bufs["grad"] = torch.empty(1, dtype=torch.float32)
    return bufs


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_every_workload_step_is_taken(floor, name):
    cfg = dict(workloads.CONFIGS[name])
    host = workloads.make(name)
    if host.T % 4 != 0:
        pytest.skip("the floor leg runs for T % 4 == 0")
    for real in (torch.float32, torch.bfloat16):
        arrays, calls = bench.workload_calls(name, cfg, host, real.itemsize)
        if real != torch.float32 and any(c[1] not in bench.BATCH_FIELDS for c in calls):
            continue   # fp32-only workloads
        bufs = _buffers(arrays, real)
        rec = bench.floor_record(calls, [bufs] * len(calls), host.num_envs, host.T)
        tiles = floor.bench_floor_prepare(ctypes.byref(rec))
        assert tiles == sum(-(-host.num_envs * host.T // 2048) for _ in calls), (name, real)
        for c in range(rec.ncalls):
            f = rec.calls[c]
            assert f.shift >= 1 and f.magic > 0
            assert f.n4 + f.n2 + f.n1 == sum(
                1 for role, a in zip(bench.FLOOR_ROLES[calls[c][1]], calls[c][2])
                if role == "in" and isinstance(a, str) and a.startswith("@"))
