"""bf16 and fp16 storage on the GPU: every estimator with its real-valued
arrays stored as bfloat16 or float16 and its arithmetic in fp32.

Bar (derived from the arithmetic): the kernel's fp32 result y meets the fp32
bar |y - o| <= 1e-4 * (1 + |o|) against the fp64 oracle o evaluated on the
same (exactly widened) inputs, and the stored output g is y rounded once to
the storage type, |g - y| <= u * |y| with unit roundoff u = 2^-8 (bf16, 8
significant bits) or 2^-11 (fp16, 11 bits).  Together:
    |g - o| <= 1e-4 * (1 + |o|) * (1 + u) + u * |o|.
The rounding itself is pinned bit for bit (round to nearest, ties to even)
against torch's conversion on sums that are exact in fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

UNIT_ROUNDOFF = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
DTYPES = [torch.bfloat16, torch.float16]
# T % 4 != 0 (windows widened to aligned starts), wave-local, eight-wave (rows
# sharing tiles), one-wave (>= 4096 rows of 257..1023 steps, with T % 4 == 0
# and not), eight-wave, 16-wave (rows of 4096+ steps), chunked (few long
# rows, with T % 4 == 0 and not: backward from 16384 steps, forward from
# 32768, and both sides of the backward 128-row bound)
SHAPES = [(5, 37), (300, 128), (33, 512), (4097, 300), (4097, 301), (9, 1024), (5, 8192),
          (3, 16400), (3, 16401), (2, 20000), (127, 16388), (128, 16388), (3, 32772),
          (3, 32773)]


def assert_lowp(gpu, ref, dtype, what):
    assert gpu.dtype == dtype, what
    g = gpu.float().cpu().numpy().astype(np.float64)
    o = np.asarray(ref, np.float64)
    assert g.shape == o.shape, what
    if g.size == 0:
        return
    u = UNIT_ROUNDOFF[dtype]
    bound = 1e-4 * (1 + np.abs(o)) * (1 + u) + u * np.abs(o)
    excess = np.abs(g - o) - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, (f"{what}: |gpu - oracle| = {abs(g[worst] - o[worst]):.3e} > "
                                f"{bound[worst]:.3e} at {worst}: gpu {g[worst]!r} "
                                f"oracle {o[worst]!r}")


def lowp(x, dtype):
    """(host array as the kernel sees it: float32 values exactly representable
    in dtype, and the device tensor of dtype)."""
    if x is None:
        return None, None
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dtype)
    return t.float().numpy(), t.cuda()


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def backward_case(op, seed, N, T, dtype):
    """(function name, device args, oracle result) for one backward estimator."""
    if op == "retrace":
        d = workloads.retrace_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
    else:
        d = workloads.backward_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
    r, r_d = lowp(d.rewards, dtype)
    v, v_d = lowp(d.q_values if op == "retrace" else d.values, dtype)
    tv, tv_d = lowp(d.trunc_values, dtype)
    b, b_d = lowp(d.bootstrap, dtype)
    term, trunc = d.terminated, d.truncated
    t_d, tr_d = dev(term), dev(trunc)
    if op == "gae":
        return ("gae", (r_d, v_d, t_d, tr_d, tv_d, b_d, 0.99, 0.95),
                oracle.gae(r, v, term, trunc, tv, b, 0.99, 0.95))
    if op == "td_lambda":
        return ("td_lambda", (r_d, v_d, t_d, tr_d, tv_d, b_d, 0.97, 0.9),
                oracle.td_lambda(r, v, term, trunc, tv, b, 0.97, 0.9))
    if op == "discounted":
        return ("discounted_returns", (r_d, t_d, tr_d, tv_d, b_d, 0.95),
                oracle.discounted_returns(r, term, trunc, tv, b, 0.95))
    mu, mu_d = lowp(d.behaviour_logp, dtype)
    pi, pi_d = lowp(d.target_logp, dtype)
    if op == "vtrace":
        return ("vtrace", (r_d, v_d, mu_d, pi_d, t_d, tr_d, tv_d, b_d, 0.99, 1.0, 1.0, 1.0),
                oracle.vtrace(r, v, mu, pi, term, trunc, tv, b, 0.99, 1.0, 1.0, 1.0))
    eq, eq_d = lowp(d.expected_q, dtype)
    return ("retrace", (r_d, v_d, eq_d, mu_d, pi_d, t_d, tr_d, tv_d, b_d, 0.99, 0.95, 1.0),
            oracle.retrace(r, v, eq, mu, pi, term, trunc, tv, b, 0.99, 0.95, 1.0))


def forward_cases(seed, N, T, dtype):
    f = workloads.forward_rollout(seed, N, T, p_start=0.05)
    x, x_d = lowp(f.increments, dtype)
    y, y_d = lowp(f.rewards, dtype)
    out = []
    for conv, flags in ((rl.RESET_ON_START, f.starts), (rl.RESET_AFTER_DONE, f.dones)):
        fl = dev(flags)
        out.append(("eligibility_traces", (x_d, fl, conv, 0.99, 0.9),
                    oracle.eligibility_traces(x, flags, conv, 0.99, 0.9)))
        out.append(("episodic_prefix_sum", (y_d, fl, conv),
                    oracle.episodic_prefix_sum(y, flags, conv)))
    rng = np.random.default_rng(seed)
    alpha = rng.standard_normal((N, T)).astype(np.float32)
    beta = rng.uniform(-0.99, 0.99, (N, T)).astype(np.float32)
    beta[rng.random((N, T)) < 0.01] = 0.0
    carry = rng.standard_normal(N).astype(np.float32)
    (a, a_d), (bt, b_d), (c, c_d) = (lowp(z, dtype) for z in (alpha, beta, carry))
    for direction in (rl.BACKWARD, rl.FORWARD):
        out.append(("affine_scan", (a_d, b_d, c_d, direction),
                    oracle.affine_scan(a, bt, c, direction)))
    return out


def outputs(x):
    return x if isinstance(x, tuple) else (x,)


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f16"])
@pytest.mark.parametrize("N,T", SHAPES)
@pytest.mark.parametrize("op", ["gae", "td_lambda", "discounted", "vtrace", "retrace"])
def test_backward_estimators_lowp(op, N, T, dtype, gpu_device):
    fn, args, ref = backward_case(op, 700 + N + T, N, T, dtype)
    got = getattr(rl, fn)(*args)
    for k, (g, o) in enumerate(zip(outputs(got), outputs(ref))):
        assert_lowp(g, o, dtype, f"{fn} out{k} N={N} T={T}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f16"])
@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_scans_lowp(N, T, dtype, gpu_device):
    for fn, args, ref in forward_cases(800 + N + T, N, T, dtype):
        assert_lowp(getattr(rl, fn)(*args), ref, dtype, f"{fn} N={N} T={T} args={args[2:]}")


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f16"])
def test_lowp_batch_matches_single_calls(dtype, gpu_device):
    # grouped launches of bf16 / fp16 members (with an f32 and an int32
    # member in between, which start groups of their own) equal single calls
    cases = [backward_case(op, 900 + i, N, T, dtype)
             for i, (op, N, T) in enumerate([("gae", 64, 128), ("vtrace", 40, 256),
                                             ("retrace", 17, 520), ("td_lambda", 5, 1024)])]
    cases += forward_cases(950, 21, 512, dtype)[:2]
    batch = rl.Batch()
    outs = [getattr(batch, fn)(*args) for fn, args, _ in cases[:3]]
    x32 = torch.randn(8, 64, device=gpu_device)
    f32_out = batch.episodic_prefix_sum(x32, torch.zeros(8, 64, dtype=torch.uint8,
                                                         device=gpu_device))
    outs += [getattr(batch, fn)(*args) for fn, args, _ in cases[3:]]
    batch.run()
    torch.cuda.synchronize(gpu_device)
    ordered = cases[:3] + cases[3:]
    for (fn, args, ref), got in zip(ordered, outs):
        single = getattr(rl, fn)(*args)
        for k, (g, s, o) in enumerate(zip(outputs(got), outputs(single), outputs(ref))):
            assert torch.equal(g, s), f"{fn} out{k}: batch and single call differ"
            assert_lowp(g, o, dtype, f"{fn} out{k} (batch)")
    assert torch.allclose(f32_out, torch.cumsum(x32, 1), atol=1e-4, rtol=1e-4)


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f16"])
def test_store_rounds_to_nearest_even(dtype, gpu_device):
    # Forward affine scan with beta = 1 at odd t and 0 elsewhere: A_t = alpha_t
    # at even t and alpha_{t-1} + alpha_t at odd t, an fp32 sum that is exact
    # (both addends are short, exponents close), so the only rounding is the
    # store.  Half of the pairs are exact ties (1 + k ulp, plus half an ulp).
    N, T = 64, 256
    rng = np.random.default_rng(5)
    eps = 2.0 ** -7 if dtype == torch.bfloat16 else 2.0 ** -10   # ulp of [1, 2)
    k = rng.integers(0, int(1 / eps), size=(N, T // 2))
    first = 1.0 + k * eps
    second = np.where(rng.random((N, T // 2)) < 0.5, eps / 2,
                      rng.integers(-64, 64, size=(N, T // 2)) * eps / 64)
    alpha = np.empty((N, T), np.float32)
    alpha[:, 0::2], alpha[:, 1::2] = first, second
    a = torch.from_numpy(alpha).to(dtype)
    assert torch.equal(a.float(), torch.from_numpy(alpha)), "inputs exact in the storage type"
    beta = torch.zeros(N, T, dtype=dtype)
    beta[:, 1::2] = 1
    out = rl.affine_scan(a.cuda(), beta.cuda(), None, rl.FORWARD).cpu()
    expect = a.float().clone()
    expect[:, 1::2] = a[:, 0::2].float() + a[:, 1::2].float()    # exact in fp32
    expect = expect.to(dtype)                                     # torch: nearest even
    assert torch.equal(out, expect)
    ties = second == eps / 2
    odd = out[:, 1::2].float().numpy()
    # a tie rounds to the neighbour with an even last bit: up from odd k
    assert np.array_equal(odd[ties], np.where(k[ties] % 2 == 1, first[ties] + eps,
                                              first[ties]))


def test_lowp_inputs_must_share_one_dtype(gpu_device):
    r = torch.zeros(4, 8, dtype=torch.bfloat16, device=gpu_device)
    v = torch.zeros(4, 8, dtype=torch.float16, device=gpu_device)
    f = torch.zeros(4, 8, dtype=torch.uint8, device=gpu_device)
    with pytest.raises(TypeError):
        rl.gae(r, v, f)
    with pytest.raises(TypeError):
        rl.gae(r.double(), r.double(), f)
