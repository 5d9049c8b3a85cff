"""Seeded synthetic rollouts shared by the tests and the benchmark.

This module only draws random numbers (numpy PCG64 via ``default_rng``); it
holds none of the estimators' arithmetic and imports neither the HIP binding
nor the oracle.  The pages measure on synthetic shape sweeps ("thousands of
environments, short rollouts"), so these draws stand in for their workloads:
rewards and values are standard normal, log-probabilities N(-1, 0.5), episode
flags are independent Bernoulli draws per step.  Draw order is fixed below so
that a seed always reproduces the same arrays.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Rollout:
    """Host arrays for one synthetic rollout window, all [num_envs, T] unless noted."""

    num_envs: int
    T: int
    rewards: np.ndarray
    values: np.ndarray
    terminated: np.ndarray          # uint8
    truncated: np.ndarray           # uint8, never set where terminated is set
    trunc_values: np.ndarray        # continuation value used at truncated steps
    bootstrap: np.ndarray           # [num_envs]
    behaviour_logp: np.ndarray
    target_logp: np.ndarray
    q_values: np.ndarray
    expected_q: np.ndarray
    params: dict = field(default_factory=dict)


@dataclass
class ForwardRollout:
    """Host arrays for the forward-time scans, all [num_envs, T]."""

    num_envs: int
    T: int
    increments: np.ndarray          # float32 ~U(0, 1): eligibility-trace increments
    rewards: np.ndarray             # float32 ~N(0, 1): prefix-sum input
    ints: np.ndarray                # int32 ~U{lo..hi}: integer prefix-sum input
    starts: np.ndarray              # uint8 episode-start flags
    dones: np.ndarray               # uint8, dones[t] = starts[t+1] (same boundaries)
    bootstrap: np.ndarray           # [num_envs]
    params: dict = field(default_factory=dict)


def _bernoulli(rng, p, shape):
    return (rng.random(shape) < p).astype(np.uint8)


def backward_rollout(seed: int, num_envs: int, T: int, p_term: float = 0.01,
                     p_trunc: float = 0.005, logp_mean: float = -1.0, logp_std: float = 0.5,
                     ratio_log_std: float = 0.5, **params) -> Rollout:
    """Rollout for the backward estimators.

    Draw order: rewards, values, bootstrap, terminated, truncated, trunc_values,
    behaviour_logp, target_logp (independent of behaviour), q_values,
    expected_q.  ``truncated`` is cleared wherever ``terminated`` is set.
    """
    rng = np.random.default_rng(seed)
    shape = (num_envs, T)
    rewards = rng.standard_normal(shape).astype(np.float32)
    values = rng.standard_normal(shape).astype(np.float32)
    bootstrap = rng.standard_normal(num_envs).astype(np.float32)
    term = _bernoulli(rng, p_term, shape)
    trunc = _bernoulli(rng, p_trunc, shape) & (1 - term)
    trunc_values = rng.standard_normal(shape).astype(np.float32)
    blogp = rng.normal(logp_mean, logp_std, shape).astype(np.float32)
    tlogp = rng.normal(logp_mean, logp_std, shape).astype(np.float32)
    q_values = rng.standard_normal(shape).astype(np.float32)
    expected_q = rng.standard_normal(shape).astype(np.float32)
    return Rollout(num_envs, T, rewards, values, term.astype(np.uint8), trunc.astype(np.uint8),
                   trunc_values, bootstrap, blogp, tlogp, q_values, expected_q, dict(params))


def retrace_rollout(seed: int, num_envs: int, T: int, p_term: float = 0.002,
                    p_trunc: float = 0.001, **params) -> Rollout:
    """Rollout for Retrace(lambda): importance ratios pi/mu = exp(N(0, 0.5)).

    Draw order: rewards, q_values, expected_q, bootstrap, terminated,
    truncated, trunc_values, behaviour_logp ~N(-1, 0.5), log-ratio ~N(0, 0.5);
    target_logp = behaviour_logp + log-ratio (in float64, then cast).
    ``values`` aliases ``q_values`` (Retrace has no state-value input).
    """
    rng = np.random.default_rng(seed)
    shape = (num_envs, T)
    rewards = rng.standard_normal(shape).astype(np.float32)
    q_values = rng.standard_normal(shape).astype(np.float32)
    expected_q = rng.standard_normal(shape).astype(np.float32)
    bootstrap = rng.standard_normal(num_envs).astype(np.float32)
    term = _bernoulli(rng, p_term, shape)
    trunc = _bernoulli(rng, p_trunc, shape) & (1 - term)
    trunc_values = rng.standard_normal(shape).astype(np.float32)
    blogp64 = rng.normal(-1.0, 0.5, shape)
    logratio = rng.normal(0.0, 0.5, shape)
    blogp = blogp64.astype(np.float32)
    tlogp = (blogp64 + logratio).astype(np.float32)
    return Rollout(num_envs, T, rewards, q_values, term.astype(np.uint8),
                   trunc.astype(np.uint8), trunc_values, bootstrap, blogp, tlogp, q_values,
                   expected_q, dict(params))


def forward_rollout(seed: int, num_envs: int, T: int, p_start: float = 0.01,
                    int_lo: int = -100, int_hi: int = 100, **params) -> ForwardRollout:
    """Rollout for the forward-time scans and the discounted-return pass that
    shares its episode boundaries.

    Draw order: rewards ~N(0, 1), increments ~U(0, 1), starts ~Bernoulli,
    bootstrap ~N(0, 1) [num_envs], ints ~U{int_lo..int_hi}.  ``dones[t]`` is
    ``starts[t+1]`` for t < T-1 and 0 at t = T-1, so the backward estimators and
    the forward scans see the same episode boundaries.
    """
    rng = np.random.default_rng(seed)
    shape = (num_envs, T)
    rewards = rng.standard_normal(shape).astype(np.float32)
    increments = rng.random(shape).astype(np.float32)
    starts = _bernoulli(rng, p_start, shape)
    bootstrap = rng.standard_normal(num_envs).astype(np.float32)
    ints = rng.integers(int_lo, int_hi + 1, size=shape, dtype=np.int64).astype(np.int32)
    dones = np.zeros(shape, np.uint8)
    if T > 1:
        dones[:, :-1] = starts[:, 1:]
    return ForwardRollout(num_envs, T, increments, rewards, ints, starts, dones, bootstrap,
                          dict(params))


# The measured workloads, with the estimator parameters each uses: the five
# configurations (seeds 1..5), the fused PPO consumers and two of few long rows.
CONFIGS = {
    "gae_8x16": dict(kind="backward", seed=1, num_envs=8, T=16, p_term=0.05, p_trunc=0.02,
                     gamma=0.99, lam=0.95),
    "gae_td_4096x128": dict(kind="backward", seed=2, num_envs=4096, T=128, p_term=0.01,
                            p_trunc=0.005, gamma=0.99, lam=0.95),
    "vtrace_4096x256": dict(kind="backward", seed=3, num_envs=4096, T=256, p_term=0.01,
                            p_trunc=0.0, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0),
    "retrace_2048x1024": dict(kind="retrace", seed=4, num_envs=2048, T=1024, p_term=0.002,
                              p_trunc=0.001, gamma=0.99, lam=0.95, c_bar=1.0),
    "forward_16384x512": dict(kind="forward", seed=5, num_envs=16384, T=512, p_start=0.01,
                              gamma=0.99, lam=0.9),
    # the fused PPO consumers on the 4096 x 128 rollout above (same seed and
    # recipe); behaviour / target log-probs serve as old / new policy
    "ppo_4096x128": dict(kind="backward", seed=2, num_envs=4096, T=128, p_term=0.01,
                         p_trunc=0.005, gamma=0.99, lam=0.95, clip_eps=0.2),
    # few long rows (the chunked path): GAE with truncation and eligibility
    # traces (x = rewards, resets after terminated steps) over one row of
    # 2^20 steps and over 8 rows of the pages' longest fused scan, 131072
    "long_1x1048576": dict(kind="backward", seed=6, num_envs=1, T=1 << 20, p_term=0.01,
                           p_trunc=0.005, gamma=0.99, lam=0.95),
    "long_8x131072": dict(kind="backward", seed=7, num_envs=8, T=131072, p_term=0.01,
                          p_trunc=0.005, gamma=0.99, lam=0.95),
}


def device_rollout(seed: int, num_envs: int, T: int, device, arrays, p_term: float = 0.001,
                   p_trunc: float = 0.0005, slab_steps: int = 1 << 28):
    """Rollout tensors drawn directly on `device` with torch's seeded generator,
    for sizes whose host copies would be unwieldy (billions of steps).  Only
    the named `arrays` are drawn, in this fixed order: rewards, values,
    trunc_values (N(0, 1)), increments (U(0, 1)), ints (int32 U{-100..100}),
    terminated (Bernoulli p_term), truncated (Bernoulli p_trunc, cleared where
    terminated), starts (Bernoulli p_term), bootstrap ([num_envs], N(0, 1)).
    Per-step arrays are drawn slab by slab of about `slab_steps` steps (whole
    rows, at least one), so the flag draws need no full-size temporaries; a
    seed, shape and slab size always give the same tensors on one device."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (num_envs, T)
    rows = max(1, slab_steps // max(1, T))
    out = {}
    for name in ("rewards", "values", "trunc_values", "increments", "ints", "terminated",
                 "truncated", "starts"):
        if name not in arrays:
            continue
        dtype = {"ints": torch.int32, "terminated": torch.uint8, "truncated": torch.uint8,
                 "starts": torch.uint8}.get(name, torch.float32)
        x = torch.empty(shape, dtype=dtype, device=device)
        for r0 in range(0, num_envs, rows):
            part = x[r0:r0 + rows]
            if name in ("rewards", "values", "trunc_values"):
                part.normal_(generator=gen)
            elif name == "increments":
                part.uniform_(generator=gen)
            elif name == "ints":
                part.random_(-100, 101, generator=gen)
            else:
                p = p_trunc if name == "truncated" else p_term
                part.copy_(torch.rand(part.shape, generator=gen, device=device) < p)
                if name == "truncated" and "terminated" in out:
                    part.masked_fill_(out["terminated"][r0:r0 + rows].bool(), 0)
        out[name] = x
    if "bootstrap" in arrays:
        out["bootstrap"] = torch.randn(num_envs, generator=gen, device=device)
    return out


def make(name: str, num_envs: int | None = None, T: int | None = None):
    """Draw the named workload; ``num_envs`` / ``T`` override the shape (same recipe)."""
    cfg = dict(CONFIGS[name])
    cfg.pop("clip_eps", None)
    kind = cfg.pop("kind")
    seed = cfg.pop("seed")
    n = cfg.pop("num_envs") if num_envs is None else (cfg.pop("num_envs"), num_envs)[1]
    t = cfg.pop("T") if T is None else (cfg.pop("T"), T)[1]
    if kind == "backward":
        return backward_rollout(seed, n, t, **cfg)
    if kind == "retrace":
        return retrace_rollout(seed, n, t, **cfg)
    return forward_rollout(seed, n, t, **cfg)
