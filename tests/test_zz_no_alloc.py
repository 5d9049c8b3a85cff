"""rlca_gae_stats_noalloc (the library's static partial-sum buffer instead of
a caller's workspace) against rlca_gae_stats on the same inputs: advantages,
returns and statistics equal bit for bit (same kernels, same reduction
order), and the statistics match the oracle's mean / std of the GPU's own
advantages to 1e-10 relative.  Consecutive calls share the buffer, so the
calls run in a row with the second smaller than the first (the buffer then
still holds the first call's extra partials, which must not be read), then
other launch shapes, then the first size again."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

# 4096 x 128: 256 partials; 300 x 77: fewer (skewed windows); then a
# one-wave shape, a chunked row pair, 16-wave workgroups (200 rows of 4100
# steps) and 16384 x 512 (the 4096-workgroup cap)
SEQUENCE = [(4096, 128, True), (300, 77, False), (4097, 301, True), (2, 20001, True),
            (200, 4100, True), (16384, 512, False), (5, 9, True), (4096, 128, True)]


def args_for(seed, N, T, trunc):
    d = workloads.backward_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    return tuple(None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
                 for x in (d.rewards, d.values, d.terminated, tr, tv, d.bootstrap))


def test_noalloc_matches_workspace_form(gpu_device):
    for i, (N, T, trunc) in enumerate(SEQUENCE):
        print(f"call {i}: {N}x{T} trunc={trunc}", flush=True)
        args = args_for(500 + i, N, T, trunc)
        adv, ret, stats = rl.gae_stats_noalloc(*args, gamma=0.99, lam=0.95)
        adv1, ret1, stats1 = rl.gae_stats(*args, gamma=0.99, lam=0.95)
        torch.cuda.synchronize()
        assert torch.equal(adv, adv1) and torch.equal(ret, ret1), f"{N}x{T}"
        assert torch.equal(stats, stats1), f"{N}x{T}: {stats.tolist()} vs {stats1.tolist()}"
        mean, std = stats.cpu().numpy()
        own_mean, own_std = oracle.mean_std(adv.cpu().numpy())
        assert mean == pytest.approx(own_mean, rel=1e-10, abs=1e-12), f"{N}x{T}"
        assert std == pytest.approx(own_std, rel=1e-10, abs=1e-12), f"{N}x{T}"


def test_noalloc_preallocated_outputs(gpu_device):
    """With advantages, returns and stats passed in, the call allocates
    nothing; back-to-back calls on one stream stay ordered."""
    N, T = 1024, 128
    args = args_for(7, N, T, True)
    adv = torch.empty(N, T, device=gpu_device)
    ret = torch.empty(N, T, device=gpu_device)
    stats = torch.empty(2, dtype=torch.float64, device=gpu_device)
    ref = rl.gae_stats(*args, gamma=0.99, lam=0.95)
    for _ in range(3):
        out = rl.gae_stats_noalloc(*args, gamma=0.99, lam=0.95, advantages=adv, returns=ret,
                                   stats=stats)
        assert out[0].data_ptr() == adv.data_ptr() and out[2].data_ptr() == stats.data_ptr()
    torch.cuda.synchronize()
    assert torch.equal(adv, ref[0]) and torch.equal(ret, ref[1]) and torch.equal(stats, ref[2])
