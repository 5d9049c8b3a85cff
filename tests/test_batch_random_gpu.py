"""Seeded random batches through rlca_run_batch: 1 to 64 calls (the limit)
of random ops and shapes (short and long rows, T % 4 != 0, few long rows
that take the chunked path, empty calls), with random truncation,
bootstrap, reset conventions and directions.  Every member is checked
against the fp64 oracle (1e-4 * (1 + |o|), int32 exact) and bit for bit
against the same call made alone, as in test_batch_gpu.py: the grouping
(classes, workgroup ranges, launches of at most 14 calls) must not change
any result."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_row_amd as rl
from tests.test_batch_gpu import Member

pytestmark = pytest.mark.gpu

OPS = ["gae", "td_lambda", "discounted", "vtrace", "retrace", "traces", "prefix", "affine"]
LENGTHS = [1, 2, 3, 4, 16, 37, 64, 127, 128, 129, 255, 256, 257, 300, 511, 512, 700, 1023,
           1024, 1025, 2047, 2048, 2049]


def random_members(rng, device):
    members = []
    for _ in range(int(rng.integers(1, 65))):
        op = str(rng.choice(OPS))
        u = rng.random()
        if u < 0.1:      # few long rows: the chunked path
            N, T = int(rng.integers(1, 9)), int(rng.integers(16384, 24000))
        elif u < 0.2:    # empty calls
            N, T = int(rng.choice([0, 3])), int(rng.choice([0, 64]))
        else:
            T = int(rng.choice(LENGTHS))
            N = int(rng.integers(1, max(2, min(5000, 2_000_000 // T))))
        kw = dict(trunc=bool(rng.random() < 0.5), boot=bool(rng.random() < 0.7))
        if op in ("traces", "prefix"):
            kw = dict(conv=int(rng.integers(0, 2)),
                      int_input=op == "prefix" and bool(rng.random() < 0.5))
        if op == "affine":
            kw = dict(direction=int(rng.integers(0, 2)), boot=bool(rng.random() < 0.5))
        members.append(Member(op, int(rng.integers(0, 1 << 30)), N, T, device, **kw))
    return members


@pytest.mark.parametrize("seed", range(16))
def test_random_batch(seed, gpu_device):
    rng = np.random.default_rng(50000 + seed)
    members = random_members(rng, gpu_device)
    batch = rl.Batch()
    for m in members:
        m.record(batch)
    batch.run()
    torch.cuda.synchronize(gpu_device)
    for m in members:
        m.check()
