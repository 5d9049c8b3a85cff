"""Chains that barely decay: beta_t at or near 1 (0.995, 0.999, 0.9999 and 1)
over zero-mean data, on rows that span waves, on every launch path (8-wave
workgroups, one wave per row, skewed windows, element-wise access, rows
longer than one tile, chunked rows), against the fp64 oracle at the parity
bar 1e-4 * (1 + |o|).

A product of n fp32 factors beta carries a relative rounding error of up to
about n * 2^-24, and it scales every value carried across the scan's waves;
with beta near 1 a chain remembers such a value over many waves, so the
error builds up (an emulation of the fp32 evaluation order gives 2e-4 at
beta = 0.999 over 2048 steps).  The library scans these calls in fp64; rows
of at most 256 steps carry nothing far and stay fp32, so they are pinned
here too.  Importance ratios are drawn at or above 1 (target log-probability
= behaviour + |N(0, 0.1)|), so V-Trace and Retrace get c_t = lambda and
beta_t = gamma * lambda exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads
from tests.test_parity_gpu import (assert_parity, check_disc, check_gae, check_retrace,
                                   check_td, check_vtrace, dev, f32)

pytestmark = pytest.mark.gpu

BETAS = [0.995, 0.999, 0.9999, 1.0]
# (N, T): 8-wave rows spanning waves; one wave per row (>= 4096 rows of
# 257..1023 steps); skewed windows (T % 4 != 0); one tile; several tiles;
# chunked (8 rows of 65536 steps); and short rows
# that stay fp32 (packed across waves, and wave-local)
SHAPES = [(64, 512), (4096, 520), (64, 1001), (48, 2048), (160, 16384), (8, 65536), (8, 65533),
          (700, 200), (512, 256)]


def rollout(seed, N, T):
    d = workloads.backward_rollout(seed, N, T, p_term=0.0005, p_trunc=0.0005)
    rng = np.random.default_rng(seed + 1)
    d.target_logp = (d.behaviour_logp + np.abs(rng.normal(0.0, 0.1, (N, T)))).astype(np.float32)
    return d


@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("N,T", SHAPES)
def test_backward_estimators(N, T, beta, gpu_device):
    d = rollout(N * 7 + T, N, T)
    what = f"{N}x{T} beta {beta}"
    check_disc(d, gpu_device, gamma=beta, what=what)
    check_gae(d, gpu_device, gamma=beta, lam=1.0, what=what)
    check_td(d, gpu_device, gamma=1.0, lam=beta, what=what)
    check_vtrace(d, gpu_device, gamma=beta, lam=1.0, what=what)
    check_retrace(d, gpu_device, gamma=1.0, lam=beta, what=what)


@pytest.mark.parametrize("beta", BETAS)
@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_and_affine(N, T, beta, gpu_device):
    f = workloads.forward_rollout(N * 11 + T, N, T, p_start=0.0005)
    what = f"{N}x{T} beta {beta}"
    x, starts = dev(f.rewards, gpu_device), dev(f.starts, gpu_device)
    e = rl.eligibility_traces(x, starts, rl.RESET_ON_START, beta, 1.0)
    assert_parity(e, oracle.eligibility_traces(f.rewards, f.starts, rl.RESET_ON_START, f32(beta),
                                               1.0), f"traces {what}")
    if beta == 1.0:
        s = rl.episodic_prefix_sum(x, starts, rl.RESET_ON_START)
        assert_parity(s, oracle.episodic_prefix_sum(f.rewards, f.starts, rl.RESET_ON_START),
                      f"prefix sum {what}")
    b = np.full((N, T), beta, np.float32)
    carry = f.bootstrap
    for direction in (rl.BACKWARD, rl.FORWARD):
        a = rl.affine_scan(x, dev(b, gpu_device), dev(carry, gpu_device), direction)
        assert_parity(a, oracle.affine_scan(f.rewards, b, carry, direction),
                      f"affine dir {direction} {what}")


@pytest.mark.parametrize("N,T", [(64, 512), (48, 2048), (160, 16384), (8, 65536)])
@pytest.mark.parametrize("gamma,lam", [(0.9995, 0.9995), (0.996, 0.97)])
def test_inexact_products(N, T, gamma, lam, gpu_device):
    """gamma * lambda is not exact in fp32 (beta near 0.999 and 0.966): the
    fp64 scans form it exactly, as the oracle does."""
    d = rollout(N * 13 + T, N, T)
    what = f"{N}x{T} gamma {gamma} lambda {lam}"
    check_gae(d, gpu_device, gamma=gamma, lam=lam, what=what)
    check_td(d, gpu_device, gamma=gamma, lam=lam, what=what)
    check_vtrace(d, gpu_device, gamma=gamma, lam=lam, c_bar=0.999, what=what)
    check_retrace(d, gpu_device, gamma=gamma, lam=lam, c_bar=0.999, what=what)
    f = workloads.forward_rollout(N * 17 + T, N, T, p_start=0.0005)
    e = rl.eligibility_traces(dev(f.rewards, gpu_device), dev(f.starts, gpu_device),
                              rl.RESET_ON_START, gamma, lam)
    assert_parity(e, oracle.eligibility_traces(f.rewards, f.starts, rl.RESET_ON_START,
                                               f32(gamma), f32(lam)), f"traces {what}")


@pytest.mark.parametrize("beta", [0.999, 1.0])
def test_element_wise_path(beta, gpu_device):
    """Inputs at different phases take the element-wise (scalar) path."""
    N, T = 64, 1000
    d = rollout(77, N, T)
    r = torch.empty(N * T + 1, device=gpu_device)[1:].view(N, T)   # phase 1
    r.copy_(dev(d.rewards, gpu_device))
    term = dev(d.terminated, gpu_device)                            # phase 0
    g = rl.discounted_returns(r, term, gamma=beta)
    assert_parity(g, oracle.discounted_returns(d.rewards, d.terminated, None, None, None,
                                               f32(beta)), f"discounted element-wise beta {beta}")


@pytest.mark.parametrize("N,T", SHAPES)
@pytest.mark.parametrize("gamma,lam", [(0.99, 1.0), (0.999, 0.95)])
def test_largest_fp32_betas(N, T, gamma, lam, gpu_device):
    """The largest beta the host still scans in fp32: 0.99 with an exact
    product, and 0.94905 (0.999 * 0.95, inexact), on every shape above, the
    tile-carry and chunked paths included, over zero-mean chains that rarely
    break."""
    d = rollout(N * 19 + T, N, T)
    what = f"{N}x{T} gamma {gamma} lambda {lam}"
    check_disc(d, gpu_device, gamma=gamma * lam, what=what)
    check_gae(d, gpu_device, gamma=gamma, lam=lam, what=what)
    check_td(d, gpu_device, gamma=gamma, lam=lam, what=what)
    check_vtrace(d, gpu_device, gamma=gamma, lam=lam, what=what)
    check_retrace(d, gpu_device, gamma=lam, lam=gamma, what=what)
    f = workloads.forward_rollout(N * 23 + T, N, T, p_start=0.0005)
    for conv in (rl.RESET_ON_START, rl.RESET_AFTER_DONE):
        flags = f.starts if conv == rl.RESET_ON_START else f.dones
        e = rl.eligibility_traces(dev(f.rewards, gpu_device), dev(flags, gpu_device), conv,
                                  gamma, lam)
        assert_parity(e, oracle.eligibility_traces(f.rewards, flags, conv, f32(gamma), f32(lam)),
                      f"traces conv {conv} {what}")
