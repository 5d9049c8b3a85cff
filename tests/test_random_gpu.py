"""Seeded random parity cases: every estimator over random shapes (including
ragged, unaligned and long rows), flag densities, discounts, clip
thresholds, reset conventions and storage types, against the fp64 oracle.
The bars are those of the fixed-shape tests: 1e-4 * (1 + |o|) for fp32
storage, plus one output rounding (u |o|, u = 2^-8 / 2^-11) for bf16 /
fp16, and bit-exact int32 sums.

Trace clips are drawn in (0, 1], the range the library accepts (it refuses
c_bar > 1, which would make the recurrence expansive), so every coefficient
|beta_t| <= 1; rho_bar, which only scales alpha, is drawn up to 2."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl

pytestmark = pytest.mark.gpu

UNIT = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def check(gpu, ref, dtype, what):
    g = gpu.float().cpu().numpy().astype(np.float64)
    o = np.asarray(ref, np.float64)
    u = UNIT[dtype]
    bound = 1e-4 * (1 + np.abs(o)) * (1 + u) + u * np.abs(o)
    bad = np.abs(g - o) > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} off, first {np.argwhere(bad)[0]}"


def place(x, dtype, rng):
    """Device tensor of x in dtype; sometimes a view starting one element
    into a larger buffer (aligned to the element size only)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dtype)
    if rng.random() < 0.3:
        buf = torch.empty(t.numel() + 1, dtype=dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t.cuda())
        return v
    return t.cuda()


def host(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).float().numpy()


@pytest.mark.parametrize("case", range(48))
def test_random_case(case, gpu_device):
    rng = np.random.default_rng(9000 + case)
    dtype = [torch.float32, torch.float32, torch.bfloat16, torch.float16][case % 4]
    kind = rng.choice(["short", "mid", "long", "few_long"])
    if kind == "short":
        N, T = int(rng.integers(1, 3000)), int(rng.integers(1, 257))
    elif kind == "mid":
        N, T = int(rng.integers(1, 5000)), int(rng.integers(257, 1100))
    elif kind == "long":
        N, T = int(rng.integers(1, 200)), int(rng.integers(1000, 5000))
    else:
        N, T = int(rng.integers(1, 160)), int(rng.integers(16384, 70000))
    p_term, p_trunc = rng.choice([0.0, 0.01, 0.2, 0.9]), rng.choice([0.0, 0.005, 0.3])
    gamma, lam = float(rng.choice([0.0, 0.5, 0.99, 1.0])), float(rng.choice([0.0, 0.9, 1.0]))
    f32 = lambda *s: rng.standard_normal(s).astype(np.float32)      # noqa: E731
    r, v, tv, eq = f32(N, T), f32(N, T), f32(N, T), f32(N, T)
    b = f32(N)
    term = (rng.random((N, T)) < p_term).astype(np.uint8)
    trunc = ((rng.random((N, T)) < p_trunc) & (term == 0)).astype(np.uint8)
    mu = rng.normal(-1, 0.5, (N, T)).astype(np.float32)
    pi = (mu + rng.normal(0, 0.7, (N, T))).astype(np.float32)
    use_trunc = rng.random() < 0.5
    tr_h, tv_h = (trunc, tv) if use_trunc else (None, None)
    what = f"case {case}: N={N} T={T} {dtype} gamma={gamma} lam={lam} trunc={use_trunc}"
    D = lambda x: None if x is None else place(x, dtype, rng)       # noqa: E731
    F = lambda x: None if x is None else torch.from_numpy(x).cuda()  # noqa: E731
    H = lambda x: None if x is None else host(x, dtype)              # noqa: E731
    op = case % 8
    if op == 0:
        adv, ret = rl.gae(D(r), D(v), F(term), F(tr_h), D(tv_h), D(b), gamma, lam)
        oa, orr = oracle.gae(H(r), H(v), term, tr_h, H(tv_h), H(b), gamma, lam)
        check(adv, oa, dtype, what)
        check(ret, orr, dtype, what)
    elif op == 1:
        check(rl.td_lambda(D(r), D(v), F(term), F(tr_h), D(tv_h), D(b), gamma, lam),
              oracle.td_lambda(H(r), H(v), term, tr_h, H(tv_h), H(b), gamma, lam), dtype, what)
    elif op == 2:
        check(rl.discounted_returns(D(r), F(term), F(tr_h), D(tv_h), D(b), gamma),
              oracle.discounted_returns(H(r), term, tr_h, H(tv_h), H(b), gamma), dtype, what)
    elif op == 3:
        rho_bar, c_bar = float(rng.choice([0.5, 1.0, 2.0])), float(rng.choice([0.5, 1.0]))
        vs, pg = rl.vtrace(D(r), D(v), D(mu), D(pi), F(term), F(tr_h), D(tv_h), D(b), gamma,
                           lam, rho_bar, c_bar)
        ovs, opg = oracle.vtrace(H(r), H(v), H(mu), H(pi), term, tr_h, H(tv_h), H(b), gamma,
                                 lam, rho_bar, c_bar)
        check(vs, ovs, dtype, what)
        check(pg, opg, dtype, what)
    elif op == 4:
        c_bar = float(rng.choice([0.5, 1.0]))
        check(rl.retrace(D(r), D(v), D(eq), D(mu), D(pi), F(term), F(tr_h), D(tv_h), D(b),
                         gamma, lam, c_bar),
              oracle.retrace(H(r), H(v), H(eq), H(mu), H(pi), term, tr_h, H(tv_h), H(b), gamma,
                             lam, c_bar), dtype, what)
    elif op == 5:
        conv = int(rng.integers(0, 2))
        x = rng.random((N, T)).astype(np.float32)
        check(rl.eligibility_traces(D(x), F(term), conv, gamma, lam),
              oracle.eligibility_traces(H(x), term, conv, gamma, lam), dtype, what)
    elif op == 6:
        conv = int(rng.integers(0, 2))
        if dtype == torch.float32 and rng.random() < 0.5:
            xi = rng.integers(-2 ** 31, 2 ** 31, (N, T), dtype=np.int64).astype(np.int32)
            got = rl.episodic_prefix_sum(torch.from_numpy(xi).cuda(), F(term), conv)
            assert np.array_equal(got.cpu().numpy(), oracle.episodic_prefix_sum(xi, term, conv)), what
        else:
            check(rl.episodic_prefix_sum(D(r), F(term), conv),
                  oracle.episodic_prefix_sum(H(r), term, conv), dtype, what)
    else:
        beta = rng.uniform(-1, 1, (N, T)).astype(np.float32)
        beta[rng.random((N, T)) < 0.05] = 0.0
        direction = int(rng.integers(0, 2))
        carry = b if rng.random() < 0.5 else None
        check(rl.affine_scan(D(r), D(beta), D(carry), direction),
              oracle.affine_scan(H(r), H(beta), H(carry), direction), dtype, what)
