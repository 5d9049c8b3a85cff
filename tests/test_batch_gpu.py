"""rlca_run_batch on the GPU: several calls validated together and enqueued as
grouped launches (calls on the vector paths) plus single launches (unaligned
or chunked calls).

Every member of a batch is checked against the fp64 oracle to the same bar as
the single-call tests (|gpu - oracle| <= 1e-4 * (1 + |oracle|), int32 exact),
and against the single-call entry point bit for bit: a grouped launch runs
each call with the tile geometry of the call's own launch (one group per
workgroup for 8-wave shapes, one per wave for one-wave shapes), and calls
that cannot join one (unaligned, chunked, or alone in its class) run their
own kernel.
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


def dev(x, device):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)


class Member:
    """One call of a mixed batch: records itself into a Batch, reruns itself
    through the single-call entry point, and knows the oracle's answer."""

    def __init__(self, op, seed, N, T, device, trunc=True, boot=True, conv=rl.RESET_ON_START,
                 direction=rl.BACKWARD, int_input=False):
        self.op, self.what = op, f"{op} N={N} T={T} seed={seed}"
        self.device = device
        tr = lambda x: x if trunc else None         # noqa: E731
        bt = lambda x: x if boot else None          # noqa: E731
        if op in ("gae", "td_lambda", "discounted", "vtrace"):
            d = workloads.backward_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
        elif op == "retrace":
            d = workloads.retrace_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
        elif op in ("traces", "prefix"):
            d = workloads.forward_rollout(seed, N, T, p_start=0.05)
        if op == "gae":
            a = (d.rewards, d.values, d.terminated, tr(d.truncated), tr(d.trunc_values),
                 bt(d.bootstrap), 0.99, 0.95)
            self.ref = oracle.gae(*a)
            self.fn = "gae"
        elif op == "td_lambda":
            a = (d.rewards, d.values, d.terminated, tr(d.truncated), tr(d.trunc_values),
                 bt(d.bootstrap), 0.97, 0.9)
            self.ref = oracle.td_lambda(*a)
            self.fn = "td_lambda"
        elif op == "discounted":
            a = (d.rewards, d.terminated, tr(d.truncated), tr(d.trunc_values),
                 bt(d.bootstrap), 0.95)
            self.ref = oracle.discounted_returns(*a)
            self.fn = "discounted_returns"
        elif op == "vtrace":
            a = (d.rewards, d.values, d.behaviour_logp, d.target_logp, d.terminated,
                 tr(d.truncated), tr(d.trunc_values), bt(d.bootstrap), 0.99, 1.0, 1.0, 1.0)
            self.ref = oracle.vtrace(*a)
            self.fn = "vtrace"
        elif op == "retrace":
            a = (d.rewards, d.q_values, d.expected_q, d.behaviour_logp, d.target_logp,
                 d.terminated, tr(d.truncated), tr(d.trunc_values), bt(d.bootstrap), 0.99,
                 0.95, 1.0)
            self.ref = oracle.retrace(*a)
            self.fn = "retrace"
        elif op == "traces":
            flags = d.starts if conv == rl.RESET_ON_START else d.dones
            a = (d.increments, flags, conv, 0.99, 0.9)
            self.ref = oracle.eligibility_traces(*a)
            self.fn = "eligibility_traces"
        elif op == "prefix":
            flags = d.starts if conv == rl.RESET_ON_START else d.dones
            a = (d.ints if int_input else d.rewards, flags, conv)
            self.ref = oracle.episodic_prefix_sum(*a)
            self.fn = "episodic_prefix_sum"
        elif op == "affine":
            rng = np.random.default_rng(seed)
            alpha = rng.standard_normal((N, T)).astype(np.float32)
            beta = rng.uniform(-0.99, 0.99, (N, T)).astype(np.float32)
            beta[rng.random((N, T)) < 0.01] = 0.0
            carry = rng.standard_normal(N).astype(np.float32)
            a = (alpha, beta, bt(carry), direction)
            self.ref = oracle.affine_scan(*a)
            self.fn = "affine_scan"
        self.args = tuple(dev(x, device) if isinstance(x, np.ndarray) else x for x in a)

    def record(self, batch):
        self.out = getattr(batch, self.fn)(*self.args)

    def single(self):
        return getattr(rl, self.fn)(*self.args)

    def outputs(self, out):
        return out if isinstance(out, tuple) else (out,)

    def check(self):
        refs = self.outputs(self.ref)
        for k, (g, r) in enumerate(zip(self.outputs(self.out), refs)):
            if g.dtype == torch.int32:
                assert np.array_equal(g.cpu().numpy(), r), f"{self.what} out{k}"
            else:
                assert_parity(g, r, f"{self.what} out{k}")
        for k, (g, s) in enumerate(zip(self.outputs(self.out), self.outputs(self.single()))):
            assert torch.equal(g, s), f"{self.what} out{k}: batch and single call differ"


def mixed_members(device):
    """Every op, both flag conventions, both affine directions; wave-local
    (T | 256), eight-wave (T >= 1024, or fewer than 4096 rows) and one-wave
    (4096 rows and more of 257..1023 steps) shapes; T % 4 != 0 (skewed
    windows, their own class, with 4-row windows of 2047-step rows), a
    chunked few-long-rows call, and an empty one."""
    return [
        Member("gae", 1, 300, 128, device),
        Member("gae", 2, 17, 48, device, trunc=False, boot=False),
        Member("td_lambda", 3, 200, 128, device),
        Member("td_lambda", 4, 9, 1024, device, trunc=False),
        Member("discounted", 5, 33, 512, device),
        Member("discounted", 6, 5, 37, device),                  # T % 4 != 0: skewed windows
        Member("vtrace", 7, 70, 256, device),
        Member("vtrace", 8, 6, 700, device, boot=False),
        Member("retrace", 9, 40, 1024, device),
        Member("retrace", 10, 3, 16400, device),                 # few long rows: chunked
        Member("traces", 11, 150, 512, device),
        Member("traces", 12, 31, 64, device, conv=rl.RESET_AFTER_DONE),
        Member("prefix", 13, 65, 128, device),
        Member("prefix", 14, 12, 2048, device, int_input=True, conv=rl.RESET_AFTER_DONE),
        Member("affine", 15, 80, 256, device, direction=rl.BACKWARD),
        Member("affine", 16, 11, 520, device, direction=rl.FORWARD, boot=False),
        Member("affine", 17, 2, 40000, device, direction=rl.FORWARD),  # chunked forward
        Member("gae", 18, 0, 128, device),                       # empty
        # one-wave members (>= 4096 rows of 257..1023 steps), the last
        # workgroup of each only partly filled
        Member("vtrace", 19, 4100, 516, device),
        Member("traces", 20, 4097, 300, device, conv=rl.RESET_AFTER_DONE),
        Member("affine", 21, 4099, 260, device, direction=rl.BACKWARD),
        # more skewed-window members (T % 4 != 0), one grouped class
        Member("gae", 22, 300, 127, device),
        Member("vtrace", 23, 70, 255, device, trunc=False),
        Member("retrace", 24, 40, 1023, device),
        Member("traces", 25, 150, 511, device, conv=rl.RESET_AFTER_DONE),
        Member("prefix", 26, 12, 2046, device, int_input=True),
        Member("affine", 27, 11, 521, device, direction=rl.FORWARD),
        Member("affine", 28, 80, 253, device, direction=rl.BACKWARD, boot=False),
        Member("traces", 29, 4100, 2047, device),                # 4-row windows
    ]


def test_mixed_batch_matches_oracle_and_single_calls(gpu_device):
    members = mixed_members(gpu_device)
    batch = rl.Batch()
    for m in members:
        m.record(batch)
    assert len(batch) == len(members)
    batch.run()
    torch.cuda.synchronize(gpu_device)
    for m in members:
        m.check()


def test_more_calls_than_one_grouped_launch_holds(gpu_device):
    # 40 vector-path calls: three grouped launches of at most 14 calls each
    ops = ["gae", "td_lambda", "discounted", "vtrace", "retrace", "traces", "prefix", "affine"]
    members = [Member(ops[i % 8], 100 + i, 5 + 7 * i, (64, 128, 256, 512, 1024)[i % 5],
                      gpu_device) for i in range(40)]
    batch = rl.Batch()
    for m in members:
        m.record(batch)
    batch.run()
    torch.cuda.synchronize(gpu_device)
    for m in members:
        m.check()


def test_batch_reruns_are_bit_identical(gpu_device):
    members = mixed_members(gpu_device)[:8]
    batch = rl.Batch()
    for m in members:
        m.record(batch)
    batch.run()
    first = [tuple(o.clone() for o in m.outputs(m.out)) for m in members]
    for m in members:
        for o in m.outputs(m.out):
            o.fill_(float("nan")) if o.dtype == torch.float32 else o.fill_(-1)
    batch.run()
    torch.cuda.synchronize(gpu_device)
    for m, f in zip(members, first):
        for o, p in zip(m.outputs(m.out), f):
            assert torch.equal(o, p), m.what


def test_cross_call_aliasing_rejected_with_real_buffers(gpu_device):
    d = workloads.backward_rollout(1, 64, 128)
    r, v, t = (dev(x, gpu_device) for x in (d.rewards, d.values, d.terminated))
    batch = rl.Batch()
    adv, _ = batch.gae(r, v, t, with_returns=False)
    # the second call reads the first call's output
    sentinel = torch.full_like(r, 7.0)
    batch.td_lambda(adv, v, t, out=sentinel)
    with pytest.raises(rl.RlcaError, match="ALIASING"):
        batch.run()
    torch.cuda.synchronize(gpu_device)
    assert torch.all(sentinel == 7.0), "a rejected batch must launch nothing"
    # adjacent but disjoint buffers are fine
    buf = torch.empty((2, 64, 128), dtype=torch.float32, device=gpu_device)
    ok = rl.Batch()
    ok.gae(r, v, t, with_returns=False, advantages=buf[0])
    ok.td_lambda(r, v, t, out=buf[1])
    ok.run()
    torch.cuda.synchronize(gpu_device)
    assert_parity(buf[0], oracle.gae(d.rewards, d.values, d.terminated, None, None, None,
                                     0.99, 0.95)[0], "adjacent gae")
    assert_parity(buf[1], oracle.td_lambda(d.rewards, d.values, d.terminated, None, None, None,
                                           0.99, 0.95), "adjacent td")


def test_batch_limits_in_the_binding(gpu_device):
    x = torch.zeros((2, 8), device=gpu_device)
    f = torch.zeros((2, 8), dtype=torch.uint8, device=gpu_device)
    batch = rl.Batch()
    for _ in range(rl.rlca.MAX_BATCH):
        batch.episodic_prefix_sum(x, f)
    with pytest.raises(ValueError):
        batch.episodic_prefix_sum(x, f)
    rl.Batch().run()                                      # an empty batch is a no-op


def test_single_member_and_one_wave_only_batches(gpu_device):
    # a lone vector-path call runs its own kernel; a batch of one-wave calls
    # (rows of 257..1023 steps) runs them one group per wave of the grouped
    # launch, with a partly filled last workgroup (num_groups not a multiple
    # of 8)
    for members in ([Member("gae", 40, 64, 128, gpu_device)],
                    [Member("retrace", 41, 4097, 300, gpu_device),
                     Member("traces", 42, 4100, 1020, gpu_device),
                     Member("affine", 43, 4101, 260, gpu_device, direction=rl.BACKWARD)]):
        batch = rl.Batch()
        for m in members:
            m.record(batch)
        batch.run()
        torch.cuda.synchronize(gpu_device)
        for m in members:
            m.check()


def test_members_off_16_byte_alignment(gpu_device):
    """Calls whose per-step inputs all sit at one phase off the 16-byte
    boundary (views at an element offset) join the grouped launch of the
    widened-window path, outputs at another phase written element by
    element; inputs at different phases run their own (scalar) kernel.  Each
    matches the oracle and its single call bit for bit."""
    def at(x, k):
        x = np.ascontiguousarray(x)
        flat = torch.zeros(x.size + 4, dtype=torch.from_numpy(x).dtype, device=gpu_device)
        flat[k:k + x.size] = torch.from_numpy(x.reshape(-1)).to(gpu_device)
        return flat[k:k + x.size].view(x.shape)

    def out_at(shape, k):
        n = int(np.prod(shape))
        return torch.zeros(n + 4, device=gpu_device)[k:k + n].view(shape)

    cases = []
    for seed, (N, T), pin, pout, mixed in [(60, (300, 128), 1, 0, False),
                                           (61, (40, 127), 2, 2, False),
                                           (62, (9, 1024), 3, 1, False),
                                           (63, (50, 200), 1, 1, True)]:
        d = workloads.backward_rollout(seed, N, T, p_term=0.05, p_trunc=0.05)
        args = (at(d.rewards, pin), at(d.values, (pin + 1) % 4 if mixed else pin),
                at(d.terminated, pin), at(d.truncated, pin), at(d.trunc_values, pin),
                dev(d.bootstrap, gpu_device), 0.99, 0.95)
        ref = oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                         d.bootstrap, 0.99, 0.95)
        cases.append((args, ref, (N, T), pout, f"gae seed={seed} phases=({pin},{pout})"))
    batch = rl.Batch()
    outs = []
    for args, ref, shape, pout, what in cases:
        a, r = out_at(shape, pout), out_at(shape, pout)
        batch.gae(*args, advantages=a, returns=r)
        outs.append((a, r))
    batch.run()
    torch.cuda.synchronize(gpu_device)
    for (args, ref, shape, pout, what), (a, r) in zip(cases, outs):
        assert_parity(a, ref[0], f"{what} adv")
        assert_parity(r, ref[1], f"{what} ret")
        a1, r1 = out_at(shape, pout), out_at(shape, pout)
        rl.gae(*args, advantages=a1, returns=r1)
        torch.cuda.synchronize(gpu_device)
        assert torch.equal(a, a1) and torch.equal(r, r1), f"{what}: batch and single call differ"
