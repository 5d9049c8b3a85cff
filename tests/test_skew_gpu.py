"""The vector path over windows widened back to aligned block boundaries:
rows of T % 4 != 0 steps, and per-step inputs that all start at one phase
(element index mod 4 of their 16-byte aligned blocks; 8-byte for 16-bit
storage, 4-byte for flags) other than 0.  Lanes read whole aligned
four-element blocks: up to three elements past a window and, for the array's
last window, past the array's end, and for inputs at a nonzero phase up to
three elements before the array's start.  Outputs at another phase than the
inputs are written element by element.

Each input here sits inside a larger buffer whose surrounding elements are NaN
(flags: set bytes; int32: a large value), so any value read from outside the
array that reached an output would show up; each output sits between
sentinels, which must survive.  Results are checked against the fp64 oracle
to the usual bar.  Shapes cover many rows per tile, one row over two tiles,
rows of 2047 steps in 4-row windows, the chunked path, and tiny T; phases
(inputs, outputs) cover (0, 0), (1, 0), (3, 3) and (2, 1).
"""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
GUARD = 8          # elements on each side; a multiple of 4 keeps arrays aligned
SENTINEL = -1536.0   # exact in fp32, bf16 and fp16

SHAPES = [(1, 1), (2, 2), (700, 3), (9, 5), (37, 37), (33, 128), (7, 131), (5, 2047), (3, 4101),
          (2, 6125), (2, 8192), (4099, 301)]
# (phase of the per-step inputs, phase of the outputs)
PHASES = [(0, 0), (1, 0), (3, 3), (2, 1)]


def guarded(x, dtype, fill, phase=0):
    """Device copy of x inside a buffer of `fill` elements: GUARD + phase
    before it (its phase: element index mod 4 from an aligned block start),
    GUARD after."""
    x = np.ascontiguousarray(x)
    n = x.size
    start = GUARD + phase
    buf = torch.full((n + start + GUARD,), fill, dtype=dtype, device="cuda")
    buf[start:start + n] = torch.from_numpy(x.reshape(-1)).to(dtype).cuda()
    view = buf[start:start + n].view(x.shape)
    assert buf.data_ptr() % (4 * buf.element_size()) == 0
    return view


class Outputs:
    """Output views between sentinels, at `phase`."""

    def __init__(self, shape, dtype=torch.float32, phase=0):
        self.n = int(np.prod(shape))
        self.dtype = dtype
        self.start = GUARD + phase
        fill = SENTINEL if dtype != torch.int32 else 0x5EED
        self.fill = fill
        self.buf = torch.full((self.n + self.start + GUARD,), fill, dtype=dtype, device="cuda")
        self.view = self.buf[self.start:self.start + self.n].view(shape)

    def check_guards(self, what):
        head, tail = self.buf[:self.start], self.buf[self.start + self.n:]
        assert torch.all(head == self.fill) and torch.all(tail == self.fill), \
            f"{what}: wrote outside its output"


def assert_parity(gpu, ref, what):
    g = gpu.detach().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err[worst] <= TOL, f"{what}: scaled error {err[worst]:.3e} at {worst}"


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("N,T", SHAPES)
def test_backward_estimators_ignore_what_surrounds_their_arrays(N, T, phases, gpu_device):
    pin, pout = phases
    nan_in = lambda x: guarded(x, torch.float32, float("nan"), pin)              # noqa: E731
    set_flags = lambda x: guarded(x.astype(np.uint8), torch.uint8, 1, pin)      # noqa: E731
    Out = lambda: Outputs((N, T), phase=pout)                                   # noqa: E731
    d = workloads.backward_rollout(7000 + N + T, N, T, p_term=0.05, p_trunc=0.05)
    q = workloads.retrace_rollout(7100 + N + T, N, T, p_term=0.05, p_trunc=0.05)
    what = f"N={N} T={T} phases={phases}"
    r, v, tv = nan_in(d.rewards), nan_in(d.values), nan_in(d.trunc_values)
    term, trunc, boot = set_flags(d.terminated), set_flags(d.truncated), nan_in(d.bootstrap)

    a, b = Out(), Out()
    rl.gae(r, v, term, trunc, tv, boot, 0.99, 0.95, advantages=a.view, returns=b.view)
    oa, ob = oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                        d.bootstrap, 0.99, 0.95)
    assert_parity(a.view, oa, f"gae adv {what}")
    assert_parity(b.view, ob, f"gae ret {what}")

    g = Out()
    rl.td_lambda(r, v, term, trunc, tv, boot, 0.97, 0.9, out=g.view)
    assert_parity(g.view, oracle.td_lambda(d.rewards, d.values, d.terminated, d.truncated,
                                           d.trunc_values, d.bootstrap, 0.97, 0.9),
                  f"td {what}")

    h = Out()
    rl.discounted_returns(r, term, trunc, tv, boot, 0.95, out=h.view)
    assert_parity(h.view, oracle.discounted_returns(d.rewards, d.terminated, d.truncated,
                                                    d.trunc_values, d.bootstrap, 0.95),
                  f"discounted {what}")

    mu, pi = nan_in(d.behaviour_logp), nan_in(d.target_logp)
    vs, pg = Out(), Out()
    rl.vtrace(r, v, mu, pi, term, trunc, tv, boot, 0.99, 0.95, 1.2, 0.9, vs=vs.view,
              pg_advantages=pg.view)
    ovs, opg = oracle.vtrace(d.rewards, d.values, d.behaviour_logp, d.target_logp,
                             d.terminated, d.truncated, d.trunc_values, d.bootstrap, 0.99, 0.95,
                             1.2, 0.9)
    assert_parity(vs.view, ovs, f"vtrace vs {what}")
    assert_parity(pg.view, opg, f"vtrace pg {what}")

    qr = Out()
    rl.retrace(nan_in(q.rewards), nan_in(q.q_values), nan_in(q.expected_q),
               nan_in(q.behaviour_logp), nan_in(q.target_logp), set_flags(q.terminated),
               set_flags(q.truncated), nan_in(q.trunc_values), nan_in(q.bootstrap), 0.99, 0.95,
               1.0, out=qr.view)
    assert_parity(qr.view, oracle.retrace(q.rewards, q.q_values, q.expected_q,
                                          q.behaviour_logp, q.target_logp, q.terminated,
                                          q.truncated, q.trunc_values, q.bootstrap, 0.99, 0.95,
                                          1.0), f"retrace {what}")
    torch.cuda.synchronize()
    for o, name in ((a, "gae adv"), (b, "gae ret"), (g, "td"), (h, "discounted"), (vs, "vs"),
                    (pg, "pg"), (qr, "retrace")):
        o.check_guards(f"{name} {what}")


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_scans_ignore_what_surrounds_their_arrays(N, T, phases, gpu_device):
    pin, pout = phases
    nan_in = lambda x: guarded(x, torch.float32, float("nan"), pin)              # noqa: E731
    set_flags = lambda x: guarded(x.astype(np.uint8), torch.uint8, 1, pin)      # noqa: E731
    f = workloads.forward_rollout(7200 + N + T, N, T, p_start=0.05)
    what = f"N={N} T={T} phases={phases}"
    outs = []
    for conv in (rl.RESET_ON_START, rl.RESET_AFTER_DONE):
        flags = f.starts if conv == rl.RESET_ON_START else f.dones
        e = Outputs((N, T), phase=pout)
        rl.eligibility_traces(nan_in(f.increments), set_flags(flags), conv, 0.99, 0.9,
                              out=e.view)
        assert_parity(e.view, oracle.eligibility_traces(f.increments, flags, conv, 0.99, 0.9),
                      f"traces conv={conv} {what}")
        s = Outputs((N, T), phase=pout)
        rl.episodic_prefix_sum(nan_in(f.rewards), set_flags(flags), conv, out=s.view)
        assert_parity(s.view, oracle.episodic_prefix_sum(f.rewards, flags, conv),
                      f"prefix f32 conv={conv} {what}")
        i = Outputs((N, T), torch.int32, phase=pout)
        rl.episodic_prefix_sum(guarded(f.ints, torch.int32, 1 << 30, pin), set_flags(flags),
                               conv, out=i.view)
        assert np.array_equal(i.view.cpu().numpy(), oracle.episodic_prefix_sum(f.ints, flags,
                                                                                conv)), \
            f"prefix i32 conv={conv} {what}"
        outs += [(e, "traces"), (s, "prefix f32"), (i, "prefix i32")]
    torch.cuda.synchronize()
    for o, name in outs:
        o.check_guards(f"{name} {what}")


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("N,T", SHAPES)
@pytest.mark.parametrize("direction", [rl.BACKWARD, rl.FORWARD])
def test_affine_scan_ignores_what_surrounds_its_arrays(N, T, direction, phases, gpu_device):
    pin, pout = phases
    nan_in = lambda x: guarded(x, torch.float32, float("nan"), pin)              # noqa: E731
    rng = np.random.default_rng(7300 + N + T + direction)
    alpha = rng.standard_normal((N, T)).astype(np.float32)
    beta = rng.uniform(-0.99, 0.99, (N, T)).astype(np.float32)
    beta[rng.random((N, T)) < 0.05] = 0.0
    carry = rng.standard_normal(N).astype(np.float32)
    out = Outputs((N, T), phase=pout)
    rl.affine_scan(nan_in(alpha), nan_in(beta), nan_in(carry), direction, out=out.view)
    what = f"affine dir={direction} N={N} T={T} phases={phases}"
    assert_parity(out.view, oracle.affine_scan(alpha, beta, carry, direction), what)
    torch.cuda.synchronize()
    out.check_guards(what)


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N,T", [(37, 37), (3, 16400), (3, 16401), (4099, 301)])
def test_lowp_storage_ignores_what_surrounds_its_arrays(N, T, dtype, phases, gpu_device):
    pin, pout = phases
    set_flags = lambda x: guarded(x.astype(np.uint8), torch.uint8, 1, pin)      # noqa: E731
    d = workloads.backward_rollout(7400 + N + T, N, T, p_term=0.05, p_trunc=0.05)
    lp = lambda x: guarded(x, dtype, float("nan"), pin)             # noqa: E731
    host = lambda x: torch.from_numpy(x).to(dtype).float().numpy()  # noqa: E731
    a, b = Outputs((N, T), dtype, pout), Outputs((N, T), dtype, pout)
    rl.gae(lp(d.rewards), lp(d.values), set_flags(d.terminated), set_flags(d.truncated),
           lp(d.trunc_values), lp(d.bootstrap), 0.99, 0.95, advantages=a.view, returns=b.view)
    oa, ob = oracle.gae(host(d.rewards), host(d.values), d.terminated, d.truncated,
                        host(d.trunc_values), host(d.bootstrap), 0.99, 0.95)
    u = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    for o, ref, name in ((a, oa, "adv"), (b, ob, "ret")):
        g = o.view.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), f"{name} N={N} T={T}: non-finite output"
        bound = 1e-4 * (1 + np.abs(ref)) * (1 + u) + u * np.abs(ref)
        assert np.all(np.abs(g - ref) <= bound), f"gae {name} {dtype} N={N} T={T}"
    torch.cuda.synchronize()
    a.check_guards(f"adv {dtype} N={N} T={T}")
    b.check_guards(f"ret {dtype} N={N} T={T}")
