"""Pins for the fp64 oracle: things other than the oracle itself that fix its values.

* brute-force unrolled sums (tests/brute.py) on tiny inputs, exhaustive over the
  per-step flag patterns (none / terminated / truncated / both);
* closed forms and textbook special cases;
* identities between estimators (GAE at lambda=0 and lambda=1, TD(lambda) as
  GAE plus values, V-Trace on-policy, Retrace at lambda=0 and on-policy);
* no-leak invariance across done steps and the window-split (carry) invariant;
* the worked four-thread scan trace of the rl-triton summary, Appendix A.
"""
import ast
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-11


def close(a, b, rtol=RTOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= rtol, f"max scaled error {err}"


def flag_patterns(T):
    """All 4^T per-step (terminated, truncated) patterns as rows."""
    pats = np.array(list(itertools.product(range(4), repeat=T)), dtype=np.uint8)
    return (pats & 1).astype(np.uint8), ((pats >> 1) & 1).astype(np.uint8)


def rand_inputs(seed, N, T):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)  # noqa: E731
    return dict(r=f(N, T), v=f(N, T), tv=f(N, T), b=f(N), q=f(N, T), eq=f(N, T),
                blogp=rng.normal(-1, 0.5, (N, T)).astype(np.float32),
                tlogp=rng.normal(-1, 0.5, (N, T)).astype(np.float32),
                x=rng.random((N, T)).astype(np.float32))


# ----------------------------------------------------------------- Appendix A


def _eval(expr, env):
    """Evaluate a +/* expression over named integers (no eval of arbitrary code)."""
    def go(node):
        if isinstance(node, ast.Expression):
            return go(node.body)
        if isinstance(node, ast.BinOp) and isinstance(node.op, ast.Add):
            return go(node.left) + go(node.right)
        if isinstance(node, ast.BinOp) and isinstance(node.op, ast.Mult):
            return go(node.left) * go(node.right)
        if isinstance(node, ast.Name):
            return env[node.id]
        raise ValueError(f"unsupported node {ast.dump(node)}")
    return go(ast.parse(expr, mode="eval"))


def combine(later, earlier_in_list):
    """The summary's operator: (aB, bB) (+) (aA, bA) = (aB + bB*aA, bA*bB)."""
    (ab, bb), (aa, ba) = later, earlier_in_list
    return (ab + bb * aa, ba * bb)


def test_appendix_a_four_thread_trace():
    g = json.load(open(os.path.join(GOLDEN, "appendix_a_four_thread_trace.json")))
    rng = np.random.default_rng(0)
    for _ in range(20):
        env = {f"a{i}": int(rng.integers(-50, 50)) for i in range(4)}
        env.update({f"b{i}": int(rng.integers(-50, 50)) for i in range(4)})
        threads = [tuple(_eval(e, env) for e in g["initial"][f"T{i}"]) for i in range(1, 5)]
        # Hillis-Steele: at stride s thread i combines its tuple with thread i-s's
        # tuple from the previous pass (all reads before writes).
        for p in range(g["passes"]):
            s = 1 << p
            prev = list(threads)
            for i in range(len(threads)):
                if i - s >= 0:
                    threads[i] = combine(prev[i], prev[i - s])
            key = f"after_pass_{p + 1}"
            for name, exprs in g[key].items():
                idx = int(name[1:]) - 1
                assert threads[idx] == tuple(_eval(e, env) for e in exprs), (key, name)


def test_combine_is_associative_exact():
    rng = np.random.default_rng(1)
    for _ in range(1000):
        x, y, z = [(int(rng.integers(-10**6, 10**6)), int(rng.integers(-10**6, 10**6)))
                   for _ in range(3)]
        assert combine(combine(x, y), z) == combine(x, combine(y, z))


def test_oracle_gae_equals_appendix_a_full_fold():
    """A 4-step row with no flags: alpha_t = delta_t, beta_t = gamma*lambda for
    t < 3 and 0 at the window edge; the trace's full fold equals A_0."""
    d = rand_inputs(2, 1, 4)
    gamma, lam = 0.9, 0.8
    r, v, b = d["r"][0].astype(float), d["v"][0].astype(float), float(d["b"][0])
    nv = [v[1], v[2], v[3], b]
    env = {f"a{t}": r[t] + gamma * nv[t] - v[t] for t in range(4)}
    env.update({f"b{t}": gamma * lam if t < 3 else 0.0 for t in range(4)})
    g = json.load(open(os.path.join(GOLDEN, "appendix_a_four_thread_trace.json")))
    full = _eval(g["after_pass_2"]["T4"][0], env)
    adv, _ = oracle.gae(d["r"], d["v"], np.zeros((1, 4), np.uint8), bootstrap=d["b"],
                        gamma=gamma, lam=lam)
    assert abs(adv[0, 0] - full) <= 1e-12 * (1 + abs(full))


# ------------------------------------------------------ brute force, exhaustive


@pytest.mark.parametrize("T", [1, 2, 5])
def test_backward_estimators_vs_brute_force_all_flag_patterns(T):
    term, trunc = flag_patterns(T)
    N = term.shape[0]
    d = rand_inputs(10 + T, N, T)
    g, lam = 0.93, 0.7
    adv, ret = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)
    badv, bret = brute.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)
    close(adv, badv)
    close(ret, bret)
    close(oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam),
          brute.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam))
    close(oracle.discounted_returns(d["r"], term, trunc, d["tv"], d["b"], g),
          brute.discounted(d["r"], term, trunc, d["tv"], d["b"], g))
    vs, pg = oracle.vtrace(d["r"], d["v"], d["blogp"], d["tlogp"], term, trunc, d["tv"],
                           d["b"], g, lam, 1.3, 0.9)
    bvs, bpg = brute.vtrace(d["r"], d["v"], d["blogp"], d["tlogp"], term, trunc, d["tv"],
                            d["b"], g, lam, 1.3, 0.9)
    close(vs, bvs)
    close(pg, bpg)
    close(oracle.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc,
                         d["tv"], d["b"], g, lam, 1.1),
          brute.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc,
                        d["tv"], d["b"], g, lam, 1.1))


@pytest.mark.parametrize("T", [1, 3, 6])
@pytest.mark.parametrize("conv", [oracle.RESET_ON_START, oracle.RESET_AFTER_DONE])
def test_forward_scans_vs_brute_force_all_flag_patterns(T, conv):
    flags = np.array(list(itertools.product(range(2), repeat=T)), dtype=np.uint8)
    N = flags.shape[0]
    d = rand_inputs(20 + T, N, T)
    close(oracle.eligibility_traces(d["x"], flags, conv, 0.97, 0.85),
          brute.eligibility(d["x"], flags, conv, 0.97, 0.85))
    close(oracle.episodic_prefix_sum(d["r"], flags, conv), brute.prefix_sum(d["r"], flags, conv))
    xi = np.random.default_rng(3).integers(-100, 101, (N, T)).astype(np.int32)
    assert np.array_equal(oracle.episodic_prefix_sum(xi, flags, conv),
                          brute.prefix_sum(xi, flags, conv))


def test_backward_vs_brute_force_random_T8():
    rng = np.random.default_rng(7)
    N, T = 64, 8
    term = (rng.random((N, T)) < 0.15).astype(np.uint8)
    trunc = (rng.random((N, T)) < 0.15).astype(np.uint8)   # overlaps term: term wins
    d = rand_inputs(8, N, T)
    g, lam = 0.99, 0.95
    close(oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)[0],
          brute.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)[0])
    close(oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam),
          brute.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam))
    close(oracle.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc,
                         d["tv"], d["b"], g, lam, 1.0),
          brute.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc,
                        d["tv"], d["b"], g, lam, 1.0))


# --------------------------------------------------------- hand special cases


def test_gae_three_step_hand_case():
    """T=3, terminated after step 1: A_2 bootstraps, A_1 has no successor,
    A_0 chains into A_1 only."""
    g, lam = 0.9, 0.5
    r = np.array([[1.0, 2.0, 3.0]], np.float32)
    v = np.array([[0.5, -1.0, 2.0]], np.float32)
    term = np.array([[0, 1, 0]], np.uint8)
    b = np.array([4.0], np.float32)
    adv, ret = oracle.gae(r, v, term, bootstrap=b, gamma=g, lam=lam)
    a2 = 3.0 + g * 4.0 - 2.0
    a1 = 2.0 - (-1.0)
    a0 = (1.0 + g * -1.0 - 0.5) + g * lam * a1
    close(adv[0], [a0, a1, a2], 1e-15)
    close(ret[0], [a0 + 0.5, a1 - 1.0, a2 + 2.0], 1e-15)


def test_last_step_flags_override_bootstrap():
    r = np.array([[1.0, 1.0]], np.float32)
    v = np.zeros((1, 2), np.float32)
    tv = np.array([[0.0, 7.0]], np.float32)
    b = np.array([100.0], np.float32)
    g = 0.5
    none = np.zeros((1, 2), np.uint8)
    last = np.array([[0, 1]], np.uint8)
    # not done: bootstrap; terminated: 0; truncated: continuation value.
    assert oracle.discounted_returns(r, none, None, None, b, g)[0, 1] == 1.0 + 0.5 * 100.0
    assert oracle.discounted_returns(r, last, None, None, b, g)[0, 1] == 1.0
    assert oracle.discounted_returns(r, none, last, tv, b, g)[0, 1] == 1.0 + 0.5 * 7.0
    # both set: terminated wins.
    assert oracle.discounted_returns(r, last, last, tv, b, g)[0, 1] == 1.0


def test_truncation_uses_continuation_not_next_value():
    d = rand_inputs(30, 4, 6)
    trunc = np.zeros((4, 6), np.uint8)
    trunc[:, 2] = 1
    term = np.zeros((4, 6), np.uint8)
    a, _ = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.9, 0.9)
    v2 = d["v"].copy()
    v2[:, 3] += 5.0                    # next episode's first value: must not reach t=2
    a2, _ = oracle.gae(d["r"], v2, term, trunc, d["tv"], d["b"], 0.9, 0.9)
    assert np.array_equal(a[:, :3], a2[:, :3])
    tv2 = d["tv"].copy()
    tv2[:, 2] += 1.0                   # continuation value: enters A_2 as gamma * 1.0
    a3, _ = oracle.gae(d["r"], d["v"], term, trunc, tv2, d["b"], 0.9, 0.9)
    close(a3[:, 2] - a[:, 2], np.full(4, 0.9), 1e-6)


def test_vtrace_log_ratio_clip():
    """One terminated step: vs = v + rho * (r - v), rho = min(rho_bar, exp(clip(l)))."""
    r = np.array([[2.0], [2.0]], np.float32)
    v = np.array([[0.5], [0.5]], np.float32)
    mu = np.array([[0.0], [0.0]], np.float32)
    pi = np.array([[9.0], [-9.0]], np.float32)
    term = np.ones((2, 1), np.uint8)
    vs, pg = oracle.vtrace(r, v, mu, pi, term, gamma=0.9, lam=1.0, rho_bar=1e3, c_bar=1e3)
    close(vs[:, 0], [0.5 + math.exp(5) * 1.5, 0.5 + math.exp(-5) * 1.5], 1e-15)
    close(pg[:, 0], [math.exp(5) * 1.5, math.exp(-5) * 1.5], 1e-15)


# ---------------------------------------------------- closed forms, identities


def test_discounted_constant_reward_closed_form():
    g, T = 0.97, 40
    r = np.ones((1, T), np.float32)
    b = np.array([3.0], np.float32)
    G = oracle.discounted_returns(r, np.zeros((1, T), np.uint8), bootstrap=b, gamma=g)
    t = np.arange(T)
    expect = (1 - g ** (T - t)) / (1 - g) + g ** (T - t) * 3.0
    close(G[0], expect, 1e-13)


def _random_flags(seed, N, T, p=0.1):
    rng = np.random.default_rng(seed)
    term = (rng.random((N, T)) < p).astype(np.uint8)
    trunc = ((rng.random((N, T)) < p) & (term == 0)).astype(np.uint8)
    return term, trunc


def test_gae_lambda_zero_is_one_step_td_error():
    d = rand_inputs(40, 16, 32)
    term, trunc = _random_flags(41, 16, 32)
    g = 0.99
    adv, _ = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, 0.0)
    G0 = oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, 0.0)
    # TD(0) target r + gamma * next value; minus V gives the TD error.
    close(adv, G0 - d["v"])
    # and spelled out directly where the chain continues:
    cont = (term == 0) & (trunc == 0)
    cont[:, -1] = False
    r64, v64 = d["r"].astype(np.float64), d["v"].astype(np.float64)
    delta = r64[:, :-1] + g * v64[:, 1:] - v64[:, :-1]
    np.testing.assert_allclose(adv[:, :-1][cont[:, :-1]], delta[cont[:, :-1]], rtol=0,
                               atol=1e-12)


def test_zero_coefficient_cuts_non_finite_values():
    """A coefficient of 0 severs the chain (summary §5 Correctness analysis: a
    step with beta = 0 composes to (alpha, 0)), NaN and infinity included:
    with lambda = 0 GAE is the one-step TD error and Retrace the expected-
    SARSA target, V-Trace's vs - V its rho-weighted TD error; with gamma = 0
    discounted returns are the rewards; with gamma * lambda = 0 the traces
    are the increments -- elementwise, non-finite entries exactly where the
    one-step values have them, however long the episode."""
    rng = np.random.default_rng(47)
    N, T = 3, 40
    r = rng.standard_normal((N, T)).astype(np.float32)
    v = rng.standard_normal((N, T)).astype(np.float32)
    eq = rng.standard_normal((N, T)).astype(np.float32)
    mu = rng.normal(-1, 0.5, (N, T)).astype(np.float32)
    pi = rng.normal(-1, 0.5, (N, T)).astype(np.float32)
    r[0, 9], v[1, 20], eq[2, 30], v[2, 5] = np.nan, np.inf, -np.inf, np.nan
    b = rng.standard_normal(N).astype(np.float32)
    term = np.zeros((N, T), np.uint8)
    g = 0.9
    r64, v64, eq64, b64 = (x.astype(np.float64) for x in (r, v, eq, b))
    nv = np.concatenate([v64[:, 1:], b64[:, None]], axis=1)    # V(s_{t+1}), bootstrap at the edge
    neq = np.concatenate([eq64[:, 1:], b64[:, None]], axis=1)
    delta = r64 + g * nv - v64
    with np.errstate(invalid="ignore"):
        adv, _ = oracle.gae(r, v, term, None, None, b, g, 0.0)
        np.testing.assert_array_equal(adv, delta)
        np.testing.assert_array_equal(oracle.retrace(r, v, eq, mu, pi, term, None, None, b, g, 0.0),
                                      r64 + g * neq)
        vs, _ = oracle.vtrace(r, v, mu, pi, term, None, None, b, g, 0.0, 1.0, 1.0)
        rho = np.minimum(1.0, np.exp(np.clip(pi.astype(np.float64) - mu, -5, 5)))
        want = rho * delta
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(vs - v64), fin)
        close((vs - v64)[fin], want[fin])
        np.testing.assert_array_equal(oracle.discounted_returns(r, term, None, None, b, 0.0), r64)
        np.testing.assert_array_equal(oracle.eligibility_traces(r, term, 0, 0.0, 0.9), r64)
        np.testing.assert_array_equal(oracle.eligibility_traces(r, term, 0, 0.9, 0.0), r64)


def test_gae_lambda_one_plus_values_is_discounted_return():
    d = rand_inputs(42, 16, 48)
    term, trunc = _random_flags(43, 16, 48)
    _, ret = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.98, 1.0)
    G = oracle.discounted_returns(d["r"], term, trunc, d["tv"], d["b"], 0.98)
    close(ret, G)


def test_td_lambda_equals_gae_return_and_limits():
    d = rand_inputs(44, 16, 48)
    term, trunc = _random_flags(45, 16, 48)
    for lam in (0.0, 0.5, 0.95, 1.0):
        _, ret = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.98, lam)
        close(oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.98, lam), ret)
    close(oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.98, 1.0),
          oracle.discounted_returns(d["r"], term, trunc, d["tv"], d["b"], 0.98))


def test_vtrace_on_policy_reduces_to_returns():
    d = rand_inputs(46, 16, 48)
    term, trunc = _random_flags(47, 16, 48)
    same = d["blogp"]
    vs, pg = oracle.vtrace(d["r"], d["v"], same, same, term, trunc, d["tv"], d["b"], 0.99,
                           1.0, 1.0, 1.0)
    close(vs, oracle.discounted_returns(d["r"], term, trunc, d["tv"], d["b"], 0.99))
    vs_l, _ = oracle.vtrace(d["r"], d["v"], same, same, term, trunc, d["tv"], d["b"], 0.99,
                            0.9, 2.0, 2.0)
    close(vs_l, oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], 0.99, 0.9))


def test_retrace_lambda_zero_and_on_policy():
    d = rand_inputs(48, 16, 48)
    term, trunc = _random_flags(49, 16, 48)
    g = 0.99
    q0 = oracle.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc,
                        d["tv"], d["b"], g, 0.0, 1.0)
    # lambda = 0: expected-SARSA target r + gamma * E_pi Q(s_{t+1}) = TD(0) on expected_q.
    close(q0, oracle.td_lambda(d["r"], d["eq"], term, trunc, d["tv"], d["b"], g, 0.0))
    # expected_q == Q and ratios >= 1 with c_bar = 1: c = lambda everywhere, so
    # Retrace is GAE's return with values := Q.
    hi = d["blogp"] + 1.0
    qr = oracle.retrace(d["r"], d["q"], d["q"], d["blogp"], hi, term, trunc, d["tv"], d["b"],
                        g, 0.9, 1.0)
    _, ret = oracle.gae(d["r"], d["q"], term, trunc, d["tv"], d["b"], g, 0.9)
    close(qr, ret)


def test_eligibility_closed_form_and_prefix_limit():
    T = 50
    x = np.ones((1, T), np.float32)
    f = np.zeros((1, T), np.uint8)
    e = oracle.eligibility_traces(x, f, oracle.RESET_ON_START, 0.9, 0.8)
    t = np.arange(T)
    close(e[0], (1 - 0.72 ** (t + 1)) / (1 - 0.72), 1e-13)
    rng = np.random.default_rng(5)
    x = rng.random((8, T)).astype(np.float32)
    f = (rng.random((8, T)) < 0.1).astype(np.uint8)
    close(oracle.eligibility_traces(x, f, 0, 1.0, 1.0), oracle.episodic_prefix_sum(x, f, 0))


def test_prefix_sum_plain_cumsum_and_wraparound():
    rng = np.random.default_rng(6)
    x = rng.integers(-100, 101, (4, 64)).astype(np.int32)
    f = np.zeros((4, 64), np.uint8)
    assert np.array_equal(oracle.episodic_prefix_sum(x, f), np.cumsum(x, axis=1, dtype=np.int32))
    big = np.full((1, 8), 2**31 - 1, np.int32)
    out = oracle.episodic_prefix_sum(big, np.zeros((1, 8), np.uint8))
    expect = (np.arange(1, 9, dtype=np.int64) * (2**31 - 1)).astype(np.uint64)
    assert np.array_equal(out[0], expect.astype(np.uint32).view(np.int32))


def test_reset_conventions_agree_on_shifted_flags():
    rng = np.random.default_rng(8)
    N, T = 8, 64
    starts = (rng.random((N, T)) < 0.1).astype(np.uint8)
    dones = np.zeros_like(starts)
    dones[:, :-1] = starts[:, 1:]
    x = rng.random((N, T)).astype(np.float32)
    close(oracle.eligibility_traces(x, starts, 0, 0.99, 0.9),
          oracle.eligibility_traces(x, dones, 1, 0.99, 0.9), 0)
    xi = rng.integers(-100, 101, (N, T)).astype(np.int32)
    assert np.array_equal(oracle.episodic_prefix_sum(xi, starts, 0),
                          oracle.episodic_prefix_sum(xi, dones, 1))


# ------------------------------------------------------------------ invariants


def test_no_leak_across_done_steps():
    d = rand_inputs(50, 8, 40)
    term = np.zeros((8, 40), np.uint8)
    trunc = np.zeros((8, 40), np.uint8)
    term[:, 17] = 1
    trunc[:4, 9] = 1
    g, lam = 0.99, 0.95
    base = [
        oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)[0],
        oracle.td_lambda(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam),
        oracle.vtrace(d["r"], d["v"], d["blogp"], d["tlogp"], term, trunc, d["tv"], d["b"],
                      g, 1.0, 1.0, 1.0)[0],
        oracle.retrace(d["r"], d["q"], d["eq"], d["blogp"], d["tlogp"], term, trunc, d["tv"],
                       d["b"], g, lam, 1.0),
    ]
    p = {k: v.copy() for k, v in d.items()}
    for k in ("r", "v", "q", "eq", "blogp", "tlogp", "tv"):
        p[k][:, 18:] += 3.0
    p["b"] += 1.0
    pert = [
        oracle.gae(p["r"], p["v"], term, trunc, p["tv"], p["b"], g, lam)[0],
        oracle.td_lambda(p["r"], p["v"], term, trunc, p["tv"], p["b"], g, lam),
        oracle.vtrace(p["r"], p["v"], p["blogp"], p["tlogp"], term, trunc, p["tv"], p["b"],
                      g, 1.0, 1.0, 1.0)[0],
        oracle.retrace(p["r"], p["q"], p["eq"], p["blogp"], p["tlogp"], term, trunc, p["tv"],
                       p["b"], g, lam, 1.0),
    ]
    for a, b in zip(base, pert):
        assert np.array_equal(a[:, :18], b[:, :18])
    # forward: inputs before a reset do not reach past it.
    starts = np.zeros((8, 40), np.uint8)
    starts[:, 11] = 1
    x = d["x"]
    x2 = x.copy()
    x2[:, :11] += 2.0
    assert np.array_equal(oracle.eligibility_traces(x, starts, 0, 0.9, 0.9)[:, 11:],
                          oracle.eligibility_traces(x2, starts, 0, 0.9, 0.9)[:, 11:])


def test_window_split_carry_invariant():
    """Discounted returns over [k, T), then over [0, k) with bootstrap := G_k,
    reproduce the full window when step k-1 is not done (the carry that lets a
    row be processed in pieces)."""
    d = rand_inputs(52, 6, 30)
    term, trunc = _random_flags(53, 6, 30, p=0.05)
    k = 13
    term[:, k - 1] = 0
    trunc[:, k - 1] = 0
    g = 0.97
    full = oracle.discounted_returns(d["r"], term, trunc, d["tv"], d["b"], g)
    tail = oracle.discounted_returns(d["r"][:, k:], term[:, k:], trunc[:, k:], d["tv"][:, k:],
                                     d["b"], g)
    head = oracle.discounted_returns(d["r"][:, :k], term[:, :k], trunc[:, :k], d["tv"][:, :k],
                                     tail[:, 0].astype(np.float32), g)
    close(tail, full[:, k:], 1e-15)
    close(head, full[:, :k], 1e-6)   # bootstrap passes through float32


# ------------------------------------------------------------ generic affine scan


@pytest.mark.parametrize("direction", [oracle.BACKWARD, oracle.FORWARD])
def test_affine_scan_vs_brute_force(direction):
    rng = np.random.default_rng(60 + direction)
    N, T = 16, 9
    alpha = rng.standard_normal((N, T)).astype(np.float32)
    beta = rng.uniform(-1.2, 1.2, (N, T)).astype(np.float32)
    beta[rng.random((N, T)) < 0.15] = 0.0
    carry = rng.standard_normal(N).astype(np.float32)
    close(oracle.affine_scan(alpha, beta, carry, direction),
          brute.affine(alpha, beta, carry, direction))
    close(oracle.affine_scan(alpha, beta, None, direction),
          brute.affine(alpha, beta, None, direction))


def test_affine_scan_special_cases():
    rng = np.random.default_rng(62)
    a = rng.standard_normal((4, 30)).astype(np.float32)
    zero = np.zeros_like(a)
    one = np.ones_like(a)
    c = rng.standard_normal(4).astype(np.float32)
    # beta = 0: A = alpha, the carry never enters
    close(oracle.affine_scan(a, zero, c, oracle.BACKWARD), a, 0)
    # beta = 1: suffix / prefix sums plus the carry
    a64 = a.astype(np.float64)
    close(oracle.affine_scan(a, one, c, oracle.BACKWARD),
          np.cumsum(a64[:, ::-1], axis=1)[:, ::-1] + c[:, None], 1e-13)
    close(oracle.affine_scan(a, one, None, oracle.FORWARD), np.cumsum(a64, axis=1), 1e-13)


def test_affine_scan_zero_beta_severs_a_nonfinite_carry():
    """[PL] §5: a step with beta = 0 composes to (alpha, 0), so nothing from
    the carried side reaches it, not even a NaN or an infinity.  Hand values,
    backward: alpha = (1, 2, 3), beta = (0.5, 0, 0.5), carry A_3 = NaN gives
    A_2 = NaN, A_1 = 2 (cut), A_0 = 1 + 0.5 * 2 = 2; forward with carry
    A_{-1} = inf and beta = (0, 0.5, 0.5): A_0 = 1, A_1 = 2.5, A_2 = 4.25."""
    a = np.array([[1.0, 2.0, 3.0]], np.float32)
    out = oracle.affine_scan(a, np.array([[0.5, 0.0, 0.5]], np.float32),
                             np.array([np.nan], np.float32), oracle.BACKWARD)
    assert out[0, 0] == 2.0 and out[0, 1] == 2.0 and np.isnan(out[0, 2])
    out = oracle.affine_scan(a, np.array([[0.0, 0.5, 0.5]], np.float32),
                             np.array([np.inf], np.float32), oracle.FORWARD)
    assert out.tolist() == [[1.0, 2.5, 4.25]]


def test_affine_scan_reproduces_the_estimators():
    """The generic scan fed with hand-built GAE coefficients gives the GAE
    oracle's advantages; forward with (x, gamma*lambda*(1 - start)) gives the
    traces.  Ties the two oracle paths together."""
    d = rand_inputs(64, 8, 40)
    term, trunc = _random_flags(65, 8, 40)
    g, lam = 0.97, 0.9
    T = 40
    r, v, tv, b = (d[k].astype(np.float64) for k in ("r", "v", "tv", "b"))
    cont = (term == 0) & (trunc == 0)
    cont[:, -1] = False
    nv = np.where(term != 0, 0.0, np.where(trunc != 0, tv, 0.0))
    nv[:, -1] = np.where((term[:, -1] == 0) & (trunc[:, -1] == 0), b, nv[:, -1])
    vnext = np.concatenate([v[:, 1:], np.zeros((8, 1))], axis=1)
    alpha = r + g * np.where(cont, vnext, nv) - v
    beta = np.where(cont, g * lam, 0.0)
    adv, _ = oracle.gae(d["r"], d["v"], term, trunc, d["tv"], d["b"], g, lam)
    # coefficients rounded to float32 on the way in
    close(oracle.affine_scan(alpha.astype(np.float32), beta.astype(np.float32), None,
                             oracle.BACKWARD), adv, 1e-5)
    starts = (np.random.default_rng(66).random((8, T)) < 0.1).astype(np.uint8)
    x = d["x"]
    bf = np.where(starts != 0, 0.0, g * lam).astype(np.float32)
    bf[:, 0] = 0.0
    close(oracle.affine_scan(x, bf, None, oracle.FORWARD),
          oracle.eligibility_traces(x, starts, 0, g, lam), 1e-6)


# ------------------------------------------------ fused consumers of the advantages


def test_mean_std_closed_forms():
    # 1..n: mean (n+1)/2, sample variance n(n+1)/12
    for n in (2, 3, 10, 1001):
        mean, std = oracle.mean_std(np.arange(1, n + 1))
        assert mean == pytest.approx((n + 1) / 2, rel=1e-15)
        assert std == pytest.approx(math.sqrt(n * (n + 1) / 12), rel=1e-14)
    assert oracle.mean_std([3.5] * 17) == (3.5, 0.0)
    assert oracle.mean_std([2.0, -1.0]) == (0.5, pytest.approx(3 / math.sqrt(2), rel=1e-15))
    assert oracle.mean_std([7.0]) == (7.0, 0.0)      # fewer than two values: std 0


def _ppo_inputs(seed, M, spread):
    rng = np.random.default_rng(seed)
    adv = rng.standard_normal(M).astype(np.float32) * 2 + 0.5
    old = rng.normal(-1.0, 0.5, M).astype(np.float32)
    new = (old + rng.normal(0.0, spread, M)).astype(np.float32)
    return adv, new, old


def test_ppo_on_policy_recovers_normalized_advantages():
    """rho = 1: the loss is -mean(A_hat), which normalization makes 0, and the
    gradient is -A_hat / M, so A_hat = -M grad must have mean 0 and sample
    std 1 (norm_eps = 0).  Pins the normalization and the gradient scale."""
    adv, _, old = _ppo_inputs(1, 500, 0.0)
    stats = oracle.mean_std(adv)
    loss, grad = oracle.ppo_clip_loss(adv, old, old, stats, 0.2, 0.0)
    a_hat = -500 * grad
    assert abs(loss) < 1e-14
    assert abs(a_hat.mean()) < 1e-13
    assert a_hat.std(ddof=1) == pytest.approx(1.0, rel=1e-13)
    assert np.allclose(a_hat, (adv.astype(np.float64) - stats[0]) / stats[1], rtol=1e-13,
                       atol=1e-13)
    # without normalization the raw advantages pass through
    loss, grad = oracle.ppo_clip_loss(adv, old, old, None, 0.2)
    assert loss == pytest.approx(-adv.astype(np.float64).mean(), rel=1e-13)


def test_ppo_normalization_adds_epsilon_to_the_std():
    """A_hat = (A - mean) / (std + eps): the epsilon is added to the standard
    deviation, not to the variance, and keeps a zero spread finite.  rho = 1,
    so the gradient is -A_hat / M.  Hand values: A = (1, 3) has mean 2 and
    sample std sqrt(2); with eps = 0.5, A_hat = (-1, 1) / (sqrt(2) + 0.5) and
    the gradient is (1, -1) / (2 (sqrt(2) + 0.5)) = +-0.26120387496374144."""
    zero = np.zeros(2, np.float32)
    loss, grad = oracle.ppo_clip_loss(np.array([1.0, 3.0], np.float32), zero, zero,
                                      (2.0, math.sqrt(2.0)), 0.2, 0.5)
    assert loss == pytest.approx(0.0, abs=1e-16)
    assert np.allclose(grad, [0.26120387496374144, -0.26120387496374144], rtol=1e-15, atol=0)
    # equal advantages: zero spread, A_hat = 0 / (0 + eps) = 0 everywhere
    const = np.full(4, 3.5, np.float32)
    loss, grad = oracle.ppo_clip_loss(const, np.zeros(4, np.float32), np.zeros(4, np.float32),
                                      (3.5, 0.0), 0.2, 1e-8)
    assert loss == 0.0 and np.array_equal(grad, np.zeros(4))


def test_ppo_clip_branches():
    """Each sign of A_hat against each side of the clip interval, eps = 0.2."""
    M = 4
    adv = np.array([1.0, 1.0, -1.0, -1.0], np.float32)
    old = np.zeros(M, np.float32)
    new = np.log(np.array([1.5, 0.5, 1.5, 0.5])).astype(np.float32)
    rho = np.exp(new.astype(np.float64))
    loss, grad = oracle.ppo_clip_loss(adv, new, old, None, 0.2)
    # A > 0: the clip caps the gain above 1.2 (no gradient); below 0.8 the
    # unclipped, smaller term is kept.  A < 0: above 1.2 the unclipped, more
    # negative term is kept; below 0.8 the clip holds the term at 0.8 A.
    terms = np.array([1.2 * 1.0, rho[1] * 1.0, rho[2] * -1.0, 0.8 * -1.0])
    assert loss == pytest.approx(-terms.mean(), rel=1e-15)
    assert np.allclose(grad, [0.0, -rho[1] / M, rho[2] / M, 0.0], rtol=1e-15, atol=0)


def test_ppo_inside_the_clip_interval_is_the_plain_surrogate():
    adv, new, old = _ppo_inputs(2, 300, 0.02)          # |ratio - 1| < 0.2 everywhere
    rho = np.exp(new.astype(np.float64) - old)
    assert np.all(np.abs(rho - 1) < 0.2)
    loss, grad = oracle.ppo_clip_loss(adv, new, old, None, 0.2)
    assert loss == pytest.approx(-(rho * adv).mean(), rel=1e-13)
    assert np.allclose(grad, -rho * adv / 300, rtol=1e-13, atol=0)


def test_ppo_gradient_matches_finite_differences():
    """Central differences of the loss in each logp_new, away from the kinks
    at the clip edges, with normalization on."""
    adv, new, old = _ppo_inputs(3, 24, 0.3)
    rho = np.exp(new.astype(np.float64) - old)
    stats = oracle.mean_std(adv)
    _, grad = oracle.ppo_clip_loss(adv, new, old, stats, 0.2, 1e-8)
    checked = 0
    for i in range(24):
        if min(abs(rho[i] - 0.8), abs(rho[i] - 1.2)) < 0.02:
            continue
        plus, minus = new.copy(), new.copy()
        plus[i] = np.float32(new[i] + np.float32(1e-3))
        minus[i] = np.float32(new[i] - np.float32(1e-3))
        h = float(plus[i]) - float(minus[i])           # the step the float inputs really take
        lp, _ = oracle.ppo_clip_loss(adv, plus, old, stats, 0.2, 1e-8)
        lm, _ = oracle.ppo_clip_loss(adv, minus, old, stats, 0.2, 1e-8)
        assert (lp - lm) / h == pytest.approx(grad[i], rel=1e-5, abs=1e-9), i
        checked += 1
    assert checked >= 18
