"""fp32 results on long chains that never break: beta = 1 over a whole row
(an episodic prefix sum without resets, discounted returns with gamma = 1 and
no episode ends), on the chunked path (8 rows) and the tile-carry path
(160 rows of 16384 steps, 320 rows of 131072), with T % 4 == 0 and
T % 4 != 0.

Rows longer than one tile carry their scan from tile to tile (and from chunk
to chunk) in fp64, so rounding no longer accumulates with the row's length:
every output meets the parity bar 1e-4 * (1 + |A|) against the fp64 oracle
up to 131072 steps, the longest fused scan on the pages ("rl-triton",
paperlayer.ai summary, §3.1 Shared scan formulation), zero-mean data
included.  A sequential fp32 evaluation (numpy's cumulative sum, one
addition per step) misses that bar on the same zero-mean rows by far.
"""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_row_amd as rl
import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _run(x, dev):
    n, t = x.shape
    flags = np.zeros((n, t), np.uint8)
    xd = torch.from_numpy(x).to(dev)
    fd = torch.from_numpy(flags).to(dev)
    prefix = rl.episodic_prefix_sum(xd, fd, rl.RESET_ON_START).cpu().numpy().astype(np.float64)
    ret = rl.discounted_returns(xd, fd, gamma=1.0).cpu().numpy().astype(np.float64)
    o_prefix = oracle.episodic_prefix_sum(x, flags, oracle.RESET_ON_START)
    o_ret = oracle.discounted_returns(x, flags, None, None, None, 1.0)
    # sequential fp32 evaluations of the same recurrences
    s_prefix = np.cumsum(x, axis=1, dtype=np.float32).astype(np.float64)
    s_ret = np.cumsum(x[:, ::-1], axis=1, dtype=np.float32)[:, ::-1].astype(np.float64)
    return [("prefix sum", prefix, o_prefix, s_prefix), ("discounted, gamma 1", ret, o_ret, s_ret)]


def _rel(g, o):
    return np.abs(g - o) / (1.0 + np.abs(o))


@pytest.mark.parametrize("N,T", [(8, 16384), (160, 16384)])
@pytest.mark.parametrize("dist", ["normal", "uniform"])
def test_long_chain_meets_the_bar(N, T, dist, gpu_device):
    rng = np.random.default_rng(1000 + N + T)
    x = (rng.standard_normal((N, T)) if dist == "normal" else rng.random((N, T))).astype(np.float32)
    for what, g, o, _ in _run(x, gpu_device):
        worst = _rel(g, o).max()
        assert worst <= TOL, f"{what} N={N} T={T} {dist}: {worst:.3e}"


@pytest.mark.parametrize("N,T", [(8, 131072), (320, 131072), (8, 131071), (320, 131071)])
def test_very_long_chain(N, T, gpu_device):
    rng = np.random.default_rng(2000 + N + T)
    positive = rng.random((N, T)).astype(np.float32)
    for what, g, o, _ in _run(positive, gpu_device):
        worst = _rel(g, o).max()
        assert worst <= TOL, f"{what} N={N} T={T} positive: {worst:.3e}"
    zero_mean = rng.standard_normal((N, T)).astype(np.float32)
    for what, g, o, s in _run(zero_mean, gpu_device):
        worst, seq = _rel(g, o).max(), _rel(s, o).max()
        print(f"{what} N={N} T={T} zero-mean: scan {worst:.3e}, sequential fp32 {seq:.3e}")
        assert worst <= TOL, f"{what} N={N} T={T} zero-mean: {worst:.3e} (sequential {seq:.3e})"
