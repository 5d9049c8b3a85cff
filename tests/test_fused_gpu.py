"""Fused consumers of the advantages on the GPU: rlca_gae_stats (GAE with the
advantage mean / std reduced in the same pass) and rlca_ppo_clip_loss (the
PPO clipped surrogate with on-the-fly normalization), against the oracle.

Bars, derived from the arithmetic:
* gae_stats' advantages and returns equal rlca_gae's bit for bit (same
  kernel body).  Its stats equal the oracle's mean / std of the GPU's own
  advantages to 1e-10 relative (the sums run in fp64).  Against the oracle's
  own advantages o (each GPU value within e_i = 1e-4 (1 + |o_i|)), the mean
  moves by at most mean(e_i) and the std by at most max(e_i) sqrt(M/(M-1)).
* ppo_clip_loss is fed exactly the oracle's inputs (the GPU advantages and
  stats).  Each fp32 term rounds a handful of times: the bound used is 16
  units in the last place of the magnitudes that enter it,
  e_t = 16 * 2^-24 * max(rho_t, 1 + eps) * (|A_hat_t| + (|A_t| + |mean|) / (std + norm_eps)),
  so |loss - oracle| <= mean(e_t), and |M grad_t - M oracle_t| <= e_t except
  where the clip decision itself is within rounding (rho_t within 1e-5 of
  1 +- eps): there either branch is correct and the GPU value must be one of
  the two.
"""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

ULP16 = 16 * 2.0 ** -24


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def rollout_args(seed, N, T, trunc=True):
    d = workloads.backward_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    host = (d.rewards, d.values, d.terminated, tr, tv, d.bootstrap)
    return host, tuple(dev(x) for x in host)


# launch shapes: T % 4 != 0 (windows widened to aligned starts), wave-local,
# eight-wave, 16-wave (up to 256 rows of 4096+ steps, T % 4 == 0 and not),
# chunked, one-wave, and chunked with T % 4 != 0; 300 rows of 4100 steps run
# the statistics at 8 waves and plain GAE at 16, whose advantages must agree
# bit for bit
SHAPES = [(7, 37), (1, 1), (2, 2), (300, 128), (4096, 128), (33, 512), (4096, 300), (9, 1024),
          (3, 4100), (200, 4100), (200, 4101), (300, 4100), (2, 20000), (4097, 301), (2, 20001)]


@pytest.mark.parametrize("N,T", SHAPES)
@pytest.mark.parametrize("trunc", [True, False])
def test_gae_stats(N, T, trunc, gpu_device):
    host, args = rollout_args(1000 + N + T, N, T, trunc)
    adv, ret, stats = rl.gae_stats(*args, gamma=0.99, lam=0.95)
    adv1, ret1 = rl.gae(*args, gamma=0.99, lam=0.95)
    assert torch.equal(adv, adv1) and torch.equal(ret, ret1)
    mean, std = stats.cpu().numpy()
    own_mean, own_std = oracle.mean_std(adv.cpu().numpy())
    assert mean == pytest.approx(own_mean, rel=1e-10, abs=1e-12)
    assert std == pytest.approx(own_std, rel=1e-10, abs=1e-12)
    o, _ = oracle.gae(*host, 0.99, 0.95)
    o_mean, o_std = oracle.mean_std(o)
    e = 1e-4 * (1 + np.abs(o))
    M = o.size
    assert abs(mean - o_mean) <= e.mean() * 1.001
    assert abs(std - o_std) <= e.max() * np.sqrt(M / max(M - 1, 1)) * 1.001


def ppo_inputs(seed, N, T):
    rng = np.random.default_rng(seed)
    old = rng.normal(-1.0, 0.5, (N, T)).astype(np.float32)
    new = (old + rng.normal(0.0, 0.3, (N, T))).astype(np.float32)
    return new, old


def check_ppo(adv, new, old, stats, clip_eps, norm_eps, loss, grad, what):
    a = adv.cpu().numpy()
    st = None if stats is None else tuple(stats.cpu().numpy())
    o_loss, o_grad = oracle.ppo_clip_loss(a, new, old, st, clip_eps, norm_eps)
    mean, std = st if st is not None else (0.0, 1.0 - norm_eps)
    scale = 1.0 / (std + norm_eps)
    a64 = a.astype(np.float64)
    a_hat = (a64 - mean) * scale if st is not None else a64
    rho = np.exp(new.astype(np.float64) - old)
    e = ULP16 * np.maximum(rho, 1 + clip_eps) * (np.abs(a_hat) + (np.abs(a64) + abs(mean)) * scale)
    got = loss.item()
    assert abs(got - o_loss) <= e.mean(), f"{what}: loss {got!r} oracle {o_loss!r}"
    if grad is None:
        return
    M = a.size
    g = grad.cpu().numpy().astype(np.float64) * M
    og = o_grad * M
    near = (np.abs(rho - (1 + clip_eps)) < 1e-5) | (np.abs(rho - (1 - clip_eps)) < 1e-5)
    ok = np.abs(g - og) <= e
    assert np.all(ok | near), f"{what}: grad off at {np.argwhere(~(ok | near))[:5].tolist()}"
    unclipped = -rho * a_hat
    both = (np.abs(g - unclipped) <= e) | (g == 0)
    assert np.all(both[near]), f"{what}: a step at the clip edge took neither branch"


@pytest.mark.parametrize("N,T", [(1, 1), (3, 5), (64, 128), (4096, 128), (17, 1001),
                                 (1024, 1024)])
@pytest.mark.parametrize("normalize", [True, False])
def test_ppo_clip_loss(N, T, normalize, gpu_device):
    host, args = rollout_args(2000 + N + T, N, T)
    adv, _, stats = rl.gae_stats(*args)
    new, old = ppo_inputs(3000 + N, N, T)
    st = stats if normalize else None
    for clip_eps in (0.2, 0.0):
        loss, grad = rl.ppo_clip_loss(adv, dev(new), dev(old), st, clip_eps, 1e-8)
        check_ppo(adv, new, old, st, clip_eps, 1e-8, loss, grad,
                  f"N={N} T={T} norm={normalize} eps={clip_eps}")
    loss2, none = rl.ppo_clip_loss(adv, dev(new), dev(old), st, 0.2, 1e-8, with_grad=False)
    assert none is None
    loss1, _ = rl.ppo_clip_loss(adv, dev(new), dev(old), st, 0.2, 1e-8)
    assert torch.equal(loss1, loss2), "the gradient output does not change the loss"


def test_ppo_unaligned_views_take_the_scalar_path(gpu_device):
    N, T = 32, 64
    host, args = rollout_args(4000, N, T)
    adv, _, stats = rl.gae_stats(*args)
    new, old = ppo_inputs(4001, N, T + 1)
    # column views starting one float in: 4-byte but not 16-byte aligned
    new_v = dev(new)[:, 1:]
    old_v = dev(old)[:, 1:]
    buf = torch.empty(N * T + 1, device=gpu_device)
    adv_v = buf[1:].view(N, T)
    adv_v.copy_(adv)
    loss, grad = rl.ppo_clip_loss(adv_v, new_v.contiguous(), old_v.contiguous(), stats)
    check_ppo(adv_v, new[:, 1:], old[:, 1:], stats, 0.2, 1e-8, loss, grad, "unaligned adv")


def test_fused_pipeline_is_deterministic(gpu_device):
    host, args = rollout_args(5000, 4096, 128)
    new, old = ppo_inputs(5001, 4096, 128)
    first = None
    for _ in range(3):
        adv, ret, stats = rl.gae_stats(*args)
        loss, grad = rl.ppo_clip_loss(adv, dev(new), dev(old), stats)
        cur = (stats.clone(), loss.clone(), grad.clone())
        if first is None:
            first = cur
        else:
            for x, y in zip(cur, first):
                assert torch.equal(x, y)
