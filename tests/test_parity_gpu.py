"""Parity of the HIP kernels (through the C ABI) with the fp64 CPU oracle.

The bar: fp32 outputs within |gpu - oracle| <= 1e-4 * (1 + |oracle|) element by
element (the rl-triton summary's §6 validation tolerance, atol = rtol = 1e-4);
the int32 prefix sum bit-exact.  Inputs are seeded synthetic rollouts; shapes
span one lane, several tiles, ragged tails, the three memory paths (4-wide
accesses with whole-row lane chunks for T % 4 == 0 and 16-byte aligned
arrays; 4-wide reads over windows widened to block boundaries for other T or
inputs all at one other phase; element accesses for inputs at different
phases), and the five measured workloads at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4


def assert_parity(gpu, ref, what=""):
    g = gpu.detach().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, what
    if g.size == 0:
        return
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err[worst] <= TOL, (f"{what}: max scaled error {err[worst]:.3e} at {worst}: "
                               f"gpu {g[worst]!r} oracle {ref[worst]!r}")


def f32(x):
    """A parameter as the library receives it (the C ABI takes fp32), for the
    oracle: like the arrays, the oracle evaluates the library's own inputs.
    (Near beta = 1 a long chain amplifies a parameter's rounding by orders of
    magnitude, so the oracle must not see a different gamma or lambda.)"""
    return float(np.float32(x))


def dev(x, device):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)


def rollout(seed, N, T, p_term=0.05, p_trunc=0.05):
    return workloads.backward_rollout(seed, N, T, p_term=p_term, p_trunc=p_trunc)


# ----------------------------------------------------------- per-estimator runs


def check_gae(d, device, trunc=True, boot=True, gamma=0.99, lam=0.95, what=""):
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    b = d.bootstrap if boot else None
    adv, ret = rl.gae(dev(d.rewards, device), dev(d.values, device), dev(d.terminated, device),
                      dev(tr, device), dev(tv, device), dev(b, device), gamma, lam)
    oadv, oret = oracle.gae(d.rewards, d.values, d.terminated, tr, tv, b, f32(gamma), f32(lam))
    assert_parity(adv, oadv, f"gae adv {what}")
    assert_parity(ret, oret, f"gae ret {what}")


def check_td(d, device, trunc=True, boot=True, gamma=0.99, lam=0.95, what=""):
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    b = d.bootstrap if boot else None
    g = rl.td_lambda(dev(d.rewards, device), dev(d.values, device), dev(d.terminated, device),
                     dev(tr, device), dev(tv, device), dev(b, device), gamma, lam)
    assert_parity(g, oracle.td_lambda(d.rewards, d.values, d.terminated, tr, tv, b, f32(gamma),
                                      f32(lam)), f"td_lambda {what}")


def check_disc(d, device, trunc=True, boot=True, gamma=0.99, what=""):
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    b = d.bootstrap if boot else None
    g = rl.discounted_returns(dev(d.rewards, device), dev(d.terminated, device),
                              dev(tr, device), dev(tv, device), dev(b, device), gamma)
    assert_parity(g, oracle.discounted_returns(d.rewards, d.terminated, tr, tv, b, f32(gamma)),
                  f"discounted {what}")


def check_vtrace(d, device, trunc=True, boot=True, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0,
                 what=""):
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    b = d.bootstrap if boot else None
    vs, pg = rl.vtrace(dev(d.rewards, device), dev(d.values, device),
                       dev(d.behaviour_logp, device), dev(d.target_logp, device),
                       dev(d.terminated, device), dev(tr, device), dev(tv, device),
                       dev(b, device), gamma, lam, rho_bar, c_bar)
    ovs, opg = oracle.vtrace(d.rewards, d.values, d.behaviour_logp, d.target_logp,
                             d.terminated, tr, tv, b, f32(gamma), f32(lam), f32(rho_bar),
                             f32(c_bar))
    assert_parity(vs, ovs, f"vtrace vs {what}")
    assert_parity(pg, opg, f"vtrace pg {what}")


def check_retrace(d, device, trunc=True, boot=True, gamma=0.99, lam=0.95, c_bar=1.0, what=""):
    tr = d.truncated if trunc else None
    tv = d.trunc_values if trunc else None
    b = d.bootstrap if boot else None
    q = rl.retrace(dev(d.rewards, device), dev(d.q_values, device), dev(d.expected_q, device),
                   dev(d.behaviour_logp, device), dev(d.target_logp, device),
                   dev(d.terminated, device), dev(tr, device), dev(tv, device), dev(b, device),
                   gamma, lam, c_bar)
    assert_parity(q, oracle.retrace(d.rewards, d.q_values, d.expected_q, d.behaviour_logp,
                                    d.target_logp, d.terminated, tr, tv, b, f32(gamma), f32(lam),
                                    f32(c_bar)), f"retrace {what}")


def check_forward(f, device, conv=rl.RESET_ON_START, gamma=0.99, lam=0.9, what=""):
    flags = f.starts if conv == rl.RESET_ON_START else f.dones
    fl = dev(flags, device)
    e = rl.eligibility_traces(dev(f.increments, device), fl, conv, gamma, lam)
    assert_parity(e, oracle.eligibility_traces(f.increments, flags, conv, f32(gamma), f32(lam)),
                  f"eligibility {what}")
    s = rl.episodic_prefix_sum(dev(f.rewards, device), fl, conv)
    assert_parity(s, oracle.episodic_prefix_sum(f.rewards, flags, conv), f"prefix f32 {what}")
    si = rl.episodic_prefix_sum(dev(f.ints, device), fl, conv)
    assert np.array_equal(si.cpu().numpy(), oracle.episodic_prefix_sum(f.ints, flags, conv)), \
        f"prefix i32 {what}"


# ------------------------------------------------------------------ shape sweep

SHAPES = [(1, 1), (3, 1), (2, 2), (5, 3), (7, 5), (8, 16), (3, 63), (2, 64), (5, 65),
          (4, 127), (9, 128), (3, 129), (2, 255), (2, 257), (1, 1023), (2, 1024), (1, 1025),
          (3, 2049), (1, 4097), (600, 7), (1030, 4), (257, 12), (5, 3001), (700, 3),
          # windows of one row of T % 4 != 0 steps over two tiles (with skew);
          # from 4096 rows of 2047 steps, windows of 4 rows over 4 tiles
          (6, 2046), (5, 2047), (4097, 2047),
          # rows of 257..1023 steps (T % 4 == 0) take one-wave workgroups from
          # 4096 rows on; with T % 4 != 0, 8-wave ones
          (4096, 260), (4099, 516), (4096, 1020), (4097, 301), (4096, 511), (4099, 1023),
          # rows longer than 2048 steps take 16-wave workgroups up to 512 rows
          # (256 with T % 4 != 0, skewed windows): one partial tile, one
          # tile, a partial second tile, several tiles; 513 (257) rows take
          # 8-wave ones
          (3, 2052), (2, 3000), (512, 2500), (513, 2500), (1, 4096), (3, 5000), (2, 8192),
          (4, 12292), (512, 4100), (513, 4100), (5, 3001), (256, 3001), (257, 3001),
          (1, 4097), (3, 5001), (2, 8195), (4, 12291), (256, 4101), (257, 4101)]


@pytest.mark.parametrize("N,T", SHAPES)
def test_backward_shape_sweep(N, T, gpu_device):
    d = rollout(100 + N * 7 + T, N, T)
    what = f"N={N} T={T}"
    for trunc in (True, False):
        check_gae(d, gpu_device, trunc=trunc, what=what)
        check_td(d, gpu_device, trunc=trunc, what=what)
        check_disc(d, gpu_device, trunc=trunc, what=what)
        check_vtrace(d, gpu_device, trunc=trunc, lam=0.9, rho_bar=1.2, c_bar=0.8, what=what)
        check_retrace(d, gpu_device, trunc=trunc, what=what)


@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_shape_sweep(N, T, gpu_device):
    f = workloads.forward_rollout(200 + N * 7 + T, N, T, p_start=0.08)
    for conv in (rl.RESET_ON_START, rl.RESET_AFTER_DONE):
        check_forward(f, gpu_device, conv, what=f"N={N} T={T} conv={conv}")


# ------------------------------------------------------------ full-size configs


def test_config_gae_8x16(gpu_device):
    c = workloads.CONFIGS["gae_8x16"]
    d = workloads.make("gae_8x16")
    check_gae(d, gpu_device, gamma=c["gamma"], lam=c["lam"], what="8x16")


@pytest.mark.parametrize("trunc", [True, False])
def test_config_gae_td_4096x128(trunc, gpu_device):
    c = workloads.CONFIGS["gae_td_4096x128"]
    d = workloads.make("gae_td_4096x128")
    check_gae(d, gpu_device, trunc=trunc, gamma=c["gamma"], lam=c["lam"], what="4096x128")
    check_td(d, gpu_device, trunc=trunc, gamma=c["gamma"], lam=c["lam"], what="4096x128")


def test_config_vtrace_4096x256(gpu_device):
    c = workloads.CONFIGS["vtrace_4096x256"]
    d = workloads.make("vtrace_4096x256")
    check_vtrace(d, gpu_device, trunc=False, gamma=c["gamma"], lam=c["lam"],
                 rho_bar=c["rho_bar"], c_bar=c["c_bar"], what="4096x256")


def test_config_retrace_2048x1024(gpu_device):
    c = workloads.CONFIGS["retrace_2048x1024"]
    d = workloads.make("retrace_2048x1024")
    check_retrace(d, gpu_device, gamma=c["gamma"], lam=c["lam"], c_bar=c["c_bar"],
                  what="2048x1024")


def test_config_forward_16384x512(gpu_device):
    c = workloads.CONFIGS["forward_16384x512"]
    f = workloads.make("forward_16384x512")
    # discounted returns over the same episode boundaries (dones[t] = starts[t+1])
    r = rl.discounted_returns(dev(f.rewards, gpu_device), dev(f.dones, gpu_device),
                              bootstrap=dev(f.bootstrap, gpu_device), gamma=c["gamma"])
    assert_parity(r, oracle.discounted_returns(f.rewards, f.dones, None, None, f.bootstrap,
                                               c["gamma"]), "16384x512 discounted")
    check_forward(f, gpu_device, rl.RESET_ON_START, c["gamma"], c["lam"], what="16384x512")
    check_forward(f, gpu_device, rl.RESET_AFTER_DONE, c["gamma"], c["lam"], what="16384x512")
    # the two reset conventions over the same boundaries: the same launch, bit for bit
    s, dn = dev(f.starts, gpu_device), dev(f.dones, gpu_device)
    x, xi = dev(f.increments, gpu_device), dev(f.ints, gpu_device)
    assert torch.equal(rl.eligibility_traces(x, s, rl.RESET_ON_START, c["gamma"], c["lam"]),
                       rl.eligibility_traces(x, dn, rl.RESET_AFTER_DONE, c["gamma"], c["lam"]))
    assert torch.equal(rl.episodic_prefix_sum(xi, s, rl.RESET_ON_START),
                       rl.episodic_prefix_sum(xi, dn, rl.RESET_AFTER_DONE))


# ------------------------------------------------------------------- edge cases


@pytest.mark.parametrize("pattern", ["none", "all_term", "all_trunc", "both", "first", "last",
                                     "alternate"])
def test_flag_patterns(pattern, gpu_device):
    N, T = 6, 70
    d = rollout(7, N, T)
    term = np.zeros((N, T), np.uint8)
    trunc = np.zeros((N, T), np.uint8)
    if pattern == "all_term":
        term[:] = 1
    elif pattern == "all_trunc":
        trunc[:] = 1
    elif pattern == "both":
        term[:] = 1
        trunc[:] = 1
    elif pattern == "first":
        term[:, 0] = 1
        trunc[:3, 0] = 1
    elif pattern == "last":
        term[:3, -1] = 1
        trunc[3:, -1] = 1
    elif pattern == "alternate":
        term[:, ::3] = 1
        trunc[:, 1::3] = 1
    d.terminated, d.truncated = term, trunc
    for boot in (True, False):
        check_gae(d, gpu_device, boot=boot, what=pattern)
        check_td(d, gpu_device, boot=boot, what=pattern)
        check_disc(d, gpu_device, boot=boot, what=pattern)
        check_vtrace(d, gpu_device, boot=boot, what=pattern)
        check_retrace(d, gpu_device, boot=boot, what=pattern)


def test_flags_as_bool_and_nonzero_bytes(gpu_device):
    d = rollout(8, 5, 40)
    r, v = dev(d.rewards, gpu_device), dev(d.values, gpu_device)
    t_u8 = dev(d.terminated, gpu_device)
    t_bool = t_u8.bool()
    t_big = (t_u8 * 200)      # any nonzero byte counts as set
    a1, _ = rl.gae(r, v, t_u8)
    a2, _ = rl.gae(r, v, t_bool)
    a3, _ = rl.gae(r, v, t_big)
    assert torch.equal(a1, a2) and torch.equal(a1, a3)


@pytest.mark.parametrize("T", [132, 131, 4100, 4097])
@pytest.mark.parametrize("shifts", [(1, 1, 1, 1, 1), (1, 2, 1, 1, 1), (0, 0, 3, 0, 0)])
def test_views_off_16_byte_alignment(T, shifts, gpu_device):
    """Inputs that are 4-byte but not 16-byte aligned (views at an element
    offset of a larger buffer) give the same results as aligned copies.  All
    at one phase (shifts (1, 1, 1, 1, 1)), the vector path reads them from
    windows widened to their block boundaries; at different phases, the
    scalar path reads them element by element."""
    N = 37
    d = rollout(9, N, T)

    def shifted(x, dtype, k):
        flat = torch.zeros(N * T + 4, dtype=dtype, device=gpu_device)
        flat[k:k + N * T] = torch.from_numpy(np.ascontiguousarray(x)).reshape(-1).to(gpu_device)
        return flat[k:k + N * T].view(N, T)

    r = shifted(d.rewards, torch.float32, shifts[0])
    v = shifted(d.values, torch.float32, shifts[1])
    term = shifted(d.terminated, torch.uint8, shifts[2])
    trunc = shifted(d.truncated, torch.uint8, shifts[3])
    tv = shifted(d.trunc_values, torch.float32, shifts[4])
    adv, ret = rl.gae(r, v, term, trunc, tv, dev(d.bootstrap, gpu_device))
    oadv, oret = oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                            d.bootstrap, 0.99, 0.95)
    assert_parity(adv, oadv, f"shifted {shifts} adv")
    assert_parity(ret, oret, f"shifted {shifts} ret")
    xi = shifted(workloads.forward_rollout(3, N, T).ints, torch.int32, shifts[0])
    fl = shifted(workloads.forward_rollout(3, N, T).starts, torch.uint8, shifts[2])
    out = rl.episodic_prefix_sum(xi, fl)
    assert np.array_equal(out.cpu().numpy(),
                          oracle.episodic_prefix_sum(xi.cpu().numpy(), fl.cpu().numpy()))


def test_no_leak_across_done_is_bit_exact_on_gpu(gpu_device):
    """beta = 0 at a done step makes everything before it independent of what
    comes after, exactly (summary §5), also in the fp32 scan."""
    N, T = 16, 3000
    d = rollout(11, N, T, p_term=0.0, p_trunc=0.0)
    d.terminated[:, 1500] = 1
    d.truncated[:, 700] = 1
    base = []
    pert = []
    for target, dd in ((base, d), (pert, None)):
        if dd is None:
            dd = rollout(11, N, T, p_term=0.0, p_trunc=0.0)
            dd.terminated, dd.truncated = d.terminated, d.truncated
            for k in ("rewards", "values", "q_values", "expected_q", "behaviour_logp",
                      "target_logp", "trunc_values"):
                getattr(dd, k)[:, 1501:] += 1.5
            dd.bootstrap = dd.bootstrap + 2.0
        r, v = dev(dd.rewards, gpu_device), dev(dd.values, gpu_device)
        te, tr = dev(dd.terminated, gpu_device), dev(dd.truncated, gpu_device)
        tv, b = dev(dd.trunc_values, gpu_device), dev(dd.bootstrap, gpu_device)
        mu, pi = dev(dd.behaviour_logp, gpu_device), dev(dd.target_logp, gpu_device)
        target.append(rl.gae(r, v, te, tr, tv, b)[0])
        target.append(rl.td_lambda(r, v, te, tr, tv, b))
        target.append(rl.discounted_returns(r, te, tr, tv, b))
        target.append(rl.vtrace(r, v, mu, pi, te, tr, tv, b)[0])
        target.append(rl.retrace(r, dev(dd.q_values, gpu_device), dev(dd.expected_q, gpu_device),
                                 mu, pi, te, tr, tv, b))
    for a, b in zip(base, pert):
        assert torch.equal(a[:, :1501], b[:, :1501])


def test_reset_conventions_agree_bitwise_on_gpu(gpu_device):
    f = workloads.forward_rollout(12, 33, 777, p_start=0.05)
    s = dev(f.starts, gpu_device)
    dn = dev(f.dones, gpu_device)
    x = dev(f.increments, gpu_device)
    assert torch.equal(rl.eligibility_traces(x, s, rl.RESET_ON_START),
                       rl.eligibility_traces(x, dn, rl.RESET_AFTER_DONE))
    xi = dev(f.ints, gpu_device)
    assert torch.equal(rl.episodic_prefix_sum(xi, s, rl.RESET_ON_START),
                       rl.episodic_prefix_sum(xi, dn, rl.RESET_AFTER_DONE))


def test_int32_prefix_sum_wraps_exactly(gpu_device):
    N, T = 3, 5000
    x = np.full((N, T), 2**31 - 7, np.int32)
    x[1] = -(2**31)
    x[2, ::2] = 123456789
    flags = np.zeros((N, T), np.uint8)
    flags[0, 2500] = 1
    out = rl.episodic_prefix_sum(dev(x, gpu_device), dev(flags, gpu_device))
    assert np.array_equal(out.cpu().numpy(), oracle.episodic_prefix_sum(x, flags))


def test_empty_inputs(gpu_device):
    for N, T in ((0, 16), (4, 0), (0, 0)):
        z = torch.zeros((N, T), device=gpu_device)
        f = torch.zeros((N, T), dtype=torch.uint8, device=gpu_device)
        adv, ret = rl.gae(z, z, f)
        assert adv.shape == (N, T) and ret.shape == (N, T)
        assert rl.episodic_prefix_sum(z.int(), f).shape == (N, T)


def test_aliasing_rejected_with_real_buffers(gpu_device):
    d = rollout(13, 4, 32)
    r, v, te = dev(d.rewards, gpu_device), dev(d.values, gpu_device), dev(d.terminated, gpu_device)
    with pytest.raises(rl.RlcaError):
        rl.gae(r, v, te, advantages=r)
    with pytest.raises(rl.RlcaError):
        rl.td_lambda(r, v, te, out=v)
    # adjacent but disjoint halves of one buffer are fine
    buf = torch.empty((2, 4, 32), device=gpu_device)
    adv, ret = rl.gae(r, v, te, advantages=buf[0], returns=buf[1])
    oadv, oret = oracle.gae(d.rewards, d.values, d.terminated, None, None, None, 0.99, 0.95)
    assert_parity(adv, oadv, "adjacent adv")
    assert_parity(ret, oret, "adjacent ret")


def test_optional_outputs_may_be_omitted(gpu_device):
    d = rollout(14, 9, 100)
    r, v, te = dev(d.rewards, gpu_device), dev(d.values, gpu_device), dev(d.terminated, gpu_device)
    adv, ret = rl.gae(r, v, te, with_returns=False)
    assert ret is None
    assert_parity(adv, oracle.gae(d.rewards, d.values, d.terminated, None, None, None,
                                  0.99, 0.95)[0], "gae adv only")
    mu, pi = dev(d.behaviour_logp, gpu_device), dev(d.target_logp, gpu_device)
    vs, pg = rl.vtrace(r, v, mu, pi, te, with_pg=False)
    assert pg is None
    assert_parity(vs, oracle.vtrace(d.rewards, d.values, d.behaviour_logp, d.target_logp,
                                    d.terminated, None, None, None, 0.99, 1.0, 1.0, 1.0)[0],
                  "vtrace vs only")


def test_extreme_log_ratios_are_clipped(gpu_device):
    d = rollout(15, 4, 50)
    d.target_logp = d.target_logp.copy()
    d.target_logp[:, ::2] += 20.0
    d.target_logp[:, 1::5] -= 20.0
    # rho_bar = 1e3 shows the +5 side through rho; c_bar = 1 the -5 side through c
    check_vtrace(d, gpu_device, rho_bar=1e3, c_bar=1.0, lam=0.5, what="clip")
    check_retrace(d, gpu_device, c_bar=1.0, lam=0.2, what="clip")


def test_repeat_calls_are_deterministic(gpu_device):
    d = rollout(16, 300, 513)
    args = [dev(x, gpu_device) for x in (d.rewards, d.values, d.terminated, d.truncated,
                                         d.trunc_values, d.bootstrap)]
    a1, _ = rl.gae(*args)
    a2, _ = rl.gae(*args)
    assert torch.equal(a1, a2)


# ------------------------------------------------- few long rows: chunked path
# Few long rows are split into chunks that run in parallel: aggregate, chunk
# carries, apply.  Backward scans chunk rows of 16384 steps or more when
# there are fewer than 128; forward scans rows of 32768 steps or more, fewer
# than 160 of them, or fewer than 208 from 65536 steps on.  Chunks span 2048
# steps for T % 4 == 0, 2040 otherwise (the last in scan order 4 to 2043).
# Shapes cover an exact multiple of the chunk, a last chunk of 1 step, a
# short last chunk in scan order, a last chunk longer than the others,
# single rows, and both sides of each row bound (127 / 128 rows backward,
# 159 / 160 and 207 / 208 forward: the second of each pair takes one
# workgroup per row).

LONG_SHAPES = [(3, 16388), (2, 16384), (3, 16385), (5, 20000), (1, 65536), (4, 20480),
               (127, 16388), (128, 16388), (127, 32768), (128, 32768),
               # T % 4 != 0: chunk starts at any offset from an aligned step
               (3, 16387), (2, 18363), (2, 18365), (5, 20001), (1, 65537), (95, 16387)]


@pytest.mark.parametrize("N,T", LONG_SHAPES)
def test_chunked_backward_estimators(N, T, gpu_device):
    d = rollout(300 + N + T, N, T, p_term=0.002, p_trunc=0.001)
    what = f"chunked N={N} T={T}"
    for trunc in (True, False):
        check_gae(d, gpu_device, trunc=trunc, what=what)
        check_td(d, gpu_device, trunc=trunc, what=what)
        check_disc(d, gpu_device, trunc=trunc, what=what)
        check_vtrace(d, gpu_device, trunc=trunc, lam=0.95, rho_bar=1.2, c_bar=0.9, what=what)
        check_retrace(d, gpu_device, trunc=trunc, what=what)


LONG_FORWARD_SHAPES = [(3, 32772), (2, 32768), (3, 32769), (5, 40000), (1, 65536), (4, 36864),
                       (159, 32772), (160, 32772), (207, 65536), (208, 65536),
                       # T % 4 != 0
                       (3, 32771), (2, 34683), (2, 34685), (5, 40001), (1, 65537), (95, 32771)]


@pytest.mark.parametrize("N,T", LONG_FORWARD_SHAPES)
def test_chunked_forward_scans(N, T, gpu_device):
    f = workloads.forward_rollout(400 + N + T, N, T, p_start=0.002)
    for conv in (rl.RESET_ON_START, rl.RESET_AFTER_DONE):
        check_forward(f, gpu_device, conv, what=f"chunked N={N} T={T} conv={conv}")


def test_chunked_no_leak_is_bit_exact(gpu_device):
    N, T = 4, 10000
    d = rollout(17, N, T, p_term=0.0, p_trunc=0.0)
    d.terminated[:, 6000] = 1
    outs = []
    for shift in (0.0, 1.5):
        r = d.rewards.copy()
        v = d.values.copy()
        r[:, 6001:] += shift
        v[:, 6001:] += shift
        adv, _ = rl.gae(dev(r, gpu_device), dev(v, gpu_device), dev(d.terminated, gpu_device),
                        bootstrap=dev(d.bootstrap + shift, gpu_device))
        outs.append(adv)
    assert torch.equal(outs[0][:, :6001], outs[1][:, :6001])


# ------------------------------------------------------------ generic affine scan


def affine_inputs(seed, N, T):
    rng = np.random.default_rng(seed)
    alpha = rng.standard_normal((N, T)).astype(np.float32)
    beta = rng.uniform(-0.99, 0.99, (N, T)).astype(np.float32)
    beta[rng.random((N, T)) < 0.01] = 0.0
    carry = rng.standard_normal(N).astype(np.float32)
    return alpha, beta, carry


@pytest.mark.parametrize("N,T", [(1, 1), (7, 5), (100, 16), (9, 128), (3, 1025), (40, 513),
                                 (3, 10000), (2, 65536)])
@pytest.mark.parametrize("direction", [rl.BACKWARD, rl.FORWARD])
def test_affine_scan(N, T, direction, gpu_device):
    alpha, beta, carry = affine_inputs(500 + N + T + direction, N, T)
    for c in (carry, None):
        out = rl.affine_scan(dev(alpha, gpu_device), dev(beta, gpu_device), dev(c, gpu_device),
                             direction)
        assert_parity(out, oracle.affine_scan(alpha, beta, c, direction),
                      f"affine N={N} T={T} dir={direction} carry={c is not None}")


# ------------------------------------------------------- 64-bit indexing, big N*T


def test_indexing_beyond_2_pow_31_steps(gpu_device):
    """2,147,486,720 steps (> 2^31): flat offsets need 64 bits, and the grid
    (capped at 2^20 workgroups) must loop over the last row groups.  Checked
    against the oracle on sampled rows at both ends and in the middle.  Inputs
    are drawn on the device with a seeded generator (about 20 GB of HBM)."""
    N, T = (1 << 21) + 3, 1024
    gen = torch.Generator(device=gpu_device)
    gen.manual_seed(77)
    r = torch.randn((N, T), generator=gen, device=gpu_device)
    flags = (torch.rand((N, T), generator=gen, device=gpu_device) < 0.01).to(torch.uint8)
    boot = torch.randn(N, generator=gen, device=gpu_device)
    rows = [0, 1, 2, N // 2, N // 2 + 1, N - 3, N - 2, N - 1]

    def sample(x):
        return x[rows].cpu().numpy()

    out = rl.discounted_returns(r, flags, bootstrap=boot)
    assert_parity(out[rows], oracle.discounted_returns(sample(r), sample(flags), None, None,
                                                       sample(boot), 0.99), "discounted 2^31+")
    rl.eligibility_traces(r, flags, rl.RESET_ON_START, 0.99, 0.9, out=out)
    assert_parity(out[rows], oracle.eligibility_traces(sample(r), sample(flags), 0, 0.99, 0.9),
                  "eligibility 2^31+")
    del out, r, flags
    torch.cuda.empty_cache()
