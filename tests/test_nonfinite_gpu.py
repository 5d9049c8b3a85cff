"""Non-finite inputs stay inside their episode segment.

A step that ends an episode (or a row end, or a reset in the forward scans)
cuts the chain: what lies beyond it never reaches the outputs on the other
side ([PL] §5: a step with beta = 0 composes to (alpha, 0)).  The kernels
keep that for NaN and infinity too, selecting instead of multiplying by zero,
so a broken step of one environment cannot spread into the previous episode
or into the other rows that share its tile.  The oracle follows the same
rule.  Here NaN and +-inf are planted in some rows (rewards, values,
log-probabilities, alpha), with episode boundaries dense enough that no
coefficient product underflows inside a segment, and every launch shape is
run: the GPU's non-finite outputs must sit exactly where the oracle's do,
the finite ones must meet the parity bar, and rows with no planted value
must be entirely finite.  A zero coefficient (lambda = 0, gamma = 0) is a
cut as well, on both sides, checked over long unbroken episodes."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

# wave-local, T % 4 != 0 (skewed windows), one-wave (>= 4096 rows), 8-wave
# rows spanning waves, chunked few long rows
SHAPES = [(300, 128), (97, 127), (4096, 300), (40, 1000), (3, 17000)]


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def plant(rng, x, rows, rate=0.01):
    """Copy of x with NaN, +inf or -inf at about `rate` of the steps of `rows`."""
    x = x.copy()
    for r in rows:
        hit = np.flatnonzero(rng.random(x.shape[1]) < rate)
        x[r, hit] = rng.choice(np.array([np.nan, np.inf, -np.inf], np.float32), hit.size)
    return x


def compare(gpu, ref, bad_rows, what):
    g = gpu.cpu().numpy().astype(np.float64)
    o = np.asarray(ref, np.float64)
    gf, of = np.isfinite(g), np.isfinite(o)
    assert np.array_equal(gf, of), (f"{what}: non-finite outputs differ at "
                                    f"{np.argwhere(gf != of)[:5].tolist()}")
    err = np.abs(g[gf] - o[gf]) / (1 + np.abs(o[gf]))
    assert err.size == 0 or err.max() <= 1e-4, f"{what}: finite outputs off by {err.max():.3e}"
    clean = np.setdiff1d(np.arange(o.shape[0]), bad_rows)
    assert np.isfinite(g[clean]).all(), f"{what}: a clean row has a non-finite output"


@pytest.mark.parametrize("N,T", SHAPES)
def test_backward_estimators_keep_nonfinite_inside_segments(N, T, gpu_device):
    rng = np.random.default_rng(N * 31 + T)
    d = workloads.backward_rollout(int(rng.integers(1 << 20)), N, T, p_term=0.05, p_trunc=0.03)
    bad = np.unique(rng.integers(0, N, max(1, N // 10)))
    r = plant(rng, d.rewards, bad)
    v = plant(rng, d.values, bad[::2])
    pi = plant(rng, d.target_logp, bad[1::2])
    args = (r, v, d.terminated, d.truncated, d.trunc_values, d.bootstrap)
    adv, ret = rl.gae(*map(dev, args), 0.99, 0.95)
    oa, orr = oracle.gae(*args, 0.99, 0.95)
    compare(adv, oa, bad, f"gae {N}x{T}")
    compare(ret, orr, bad, f"gae returns {N}x{T}")
    compare(rl.td_lambda(*map(dev, args), 0.99, 0.95), oracle.td_lambda(*args, 0.99, 0.95), bad,
            f"td_lambda {N}x{T}")
    dargs = (r, d.terminated, d.truncated, d.trunc_values, d.bootstrap)
    compare(rl.discounted_returns(*map(dev, dargs), 0.99),
            oracle.discounted_returns(*dargs, 0.99), bad, f"discounted {N}x{T}")
    vargs = (r, v, d.behaviour_logp, pi, d.terminated, d.truncated, d.trunc_values, d.bootstrap)
    vs, pg = rl.vtrace(*map(dev, vargs), 0.99, 0.9, 1.0, 1.0)
    ovs, opg = oracle.vtrace(*vargs, 0.99, 0.9, 1.0, 1.0)
    compare(vs, ovs, bad, f"vtrace vs {N}x{T}")
    compare(pg, opg, bad, f"vtrace pg {N}x{T}")
    rargs = (r, v, d.trunc_values, d.behaviour_logp, pi, d.terminated, d.truncated,
             d.trunc_values, d.bootstrap)
    compare(rl.retrace(*map(dev, rargs), 0.99, 0.95, 1.0),
            oracle.retrace(*rargs, 0.99, 0.95, 1.0), bad, f"retrace {N}x{T}")


@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_scans_keep_nonfinite_inside_segments(N, T, gpu_device):
    rng = np.random.default_rng(N * 37 + T)
    f = workloads.forward_rollout(int(rng.integers(1 << 20)), N, T, p_start=0.05)
    bad = np.unique(rng.integers(0, N, max(1, N // 10)))
    x = plant(rng, f.increments, bad)
    for conv in (rl.RESET_ON_START, rl.RESET_AFTER_DONE):
        flags = f.starts if conv == rl.RESET_ON_START else f.dones
        compare(rl.eligibility_traces(dev(x), dev(flags), conv, 0.99, 0.9),
                oracle.eligibility_traces(x, flags, conv, 0.99, 0.9), bad,
                f"traces {N}x{T} conv {conv}")
        compare(rl.episodic_prefix_sum(dev(x), dev(flags), conv),
                oracle.episodic_prefix_sum(x, flags, conv), bad, f"prefix {N}x{T} conv {conv}")


@pytest.mark.parametrize("N,T", SHAPES)
@pytest.mark.parametrize("direction", [rl.BACKWARD, rl.FORWARD])
def test_affine_scan_zero_beta_severs_nonfinite(N, T, direction, gpu_device):
    rng = np.random.default_rng(N * 41 + T + direction)
    alpha = rng.standard_normal((N, T)).astype(np.float32)
    beta = rng.uniform(-0.99, 0.99, (N, T)).astype(np.float32)
    beta[rng.random((N, T)) < 0.05] = 0.0
    bad = np.unique(rng.integers(0, N, max(1, N // 10)))
    alpha = plant(rng, alpha, bad)
    carry = rng.standard_normal(N).astype(np.float32)
    carry[bad[:1]] = np.nan   # a non-finite carry only reaches its row's first segment
    compare(rl.affine_scan(dev(alpha), dev(beta), dev(carry), direction),
            oracle.affine_scan(alpha, beta, carry, direction), bad, f"affine {N}x{T} dir {direction}")


@pytest.mark.parametrize("N,T", SHAPES)
def test_zero_coefficients_cut_nonfinite(N, T, gpu_device):
    """lambda = 0 or gamma = 0: every step's coefficient is 0, so a NaN or
    infinity reaches no other step through the chain, even inside one long
    episode (episode ends at 0.1% of the steps)."""
    rng = np.random.default_rng(N * 43 + T)
    d = workloads.backward_rollout(int(rng.integers(1 << 20)), N, T, p_term=0.001,
                                   p_trunc=0.0005)
    bad = np.unique(rng.integers(0, N, max(1, N // 10)))
    r = plant(rng, d.rewards, bad)
    v = plant(rng, d.values, bad[::2])
    args = (r, v, d.terminated, d.truncated, d.trunc_values, d.bootstrap)
    adv, _ = rl.gae(*map(dev, args), 0.99, 0.0)
    compare(adv, oracle.gae(*args, 0.99, 0.0)[0], bad, f"gae lambda 0 {N}x{T}")
    dargs = (r, d.terminated, d.truncated, d.trunc_values, d.bootstrap)
    compare(rl.discounted_returns(*map(dev, dargs), 0.0),
            oracle.discounted_returns(*dargs, 0.0), bad, f"discounted gamma 0 {N}x{T}")
    vargs = (r, v, d.behaviour_logp, d.target_logp, d.terminated, d.truncated, d.trunc_values,
             d.bootstrap)
    vs, pg = rl.vtrace(*map(dev, vargs), 0.99, 0.0, 1.0, 1.0)
    ovs, opg = oracle.vtrace(*vargs, 0.99, 0.0, 1.0, 1.0)
    compare(vs, ovs, bad, f"vtrace lambda 0 {N}x{T}")
    compare(pg, opg, bad, f"vtrace pg lambda 0 {N}x{T}")
    rargs = (r, v, d.trunc_values, d.behaviour_logp, d.target_logp, d.terminated, d.truncated,
             d.trunc_values, d.bootstrap)
    compare(rl.retrace(*map(dev, rargs), 0.99, 0.0, 1.0),
            oracle.retrace(*rargs, 0.99, 0.0, 1.0), bad, f"retrace lambda 0 {N}x{T}")
    f = workloads.forward_rollout(int(rng.integers(1 << 20)), N, T, p_start=0.001)
    x = plant(rng, f.increments, bad)
    compare(rl.eligibility_traces(dev(x), dev(f.starts), rl.RESET_ON_START, 0.99, 0.0),
            oracle.eligibility_traces(x, f.starts, rl.RESET_ON_START, 0.99, 0.0), bad,
            f"traces lambda 0 {N}x{T}")
