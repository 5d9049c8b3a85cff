"""The chunked path's hand-off values across calls that reuse their buffers.

A chunked call passes each chunk's map and carry between its three launches
through the chunk's first output elements.  Here the same output tensors
serve call after call, alternating shapes whose chunk slots sit at
different elements, so every slot's memory holds another call's outputs or
hand-off words before it is written again.  Every call of every round must
equal the oracle at the parity bar (storage-type rounding included).  One
earlier run saw a wrong carry at a chunk boundary once (bf16, 3 x 16401);
the hand-off words are now written and read as agent-scope atomics, and this
test repeats that pattern."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

U = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
# GAE chunks all four; eligibility traces (chunked from 32768 steps) the last two
SHAPES = [(3, 16401), (3, 16400), (2, 32769), (5, 34683)]


def check(gpu, ref, dtype, what):
    g = gpu.float().cpu().numpy().astype(np.float64)
    o = np.asarray(ref, np.float64)
    u = U[dtype]
    excess = np.abs(g - o) - (1e-4 * (1 + np.abs(o)) * (1 + u) + u * np.abs(o))
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, f"{what}: gpu {g[worst]!r} oracle {o[worst]!r} at {worst}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_chunked_calls_reusing_buffers(dtype, gpu_device):
    cases = []
    for k, (N, T) in enumerate(SHAPES):
        d = workloads.backward_rollout(600 + k, N, T, p_term=0.002, p_trunc=0.001)
        host = {n: torch.from_numpy(np.ascontiguousarray(getattr(d, n))).to(dtype).float().numpy()
                for n in ("rewards", "values", "trunc_values", "bootstrap")}
        dev = {n: torch.from_numpy(h).to(dtype).to(gpu_device) for n, h in host.items()}
        flags = {n: torch.from_numpy(getattr(d, n)).to(gpu_device) for n in ("terminated",
                                                                          "truncated")}
        oa, orr = oracle.gae(host["rewards"], host["values"], d.terminated, d.truncated,
                             host["trunc_values"], host["bootstrap"], float(np.float32(0.99)),
                             float(np.float32(0.95)))
        x = torch.from_numpy(np.ascontiguousarray(host["rewards"])).to(dtype).to(gpu_device)
        ot = oracle.eligibility_traces(host["rewards"], d.terminated, oracle.RESET_AFTER_DONE,
                                       float(np.float32(0.99)), float(np.float32(0.9)))
        cases.append((N, T, dev, flags, oa, orr, x, ot))
    # one pair of output buffers for every shape: views of the same storage
    most = max(N * T for N, T, *_ in cases)
    adv_store = torch.empty(most, dtype=dtype, device=gpu_device)
    ret_store = torch.empty(most, dtype=dtype, device=gpu_device)
    for rnd in range(4):
        for N, T, dev, flags, oa, orr, x, ot in cases:
            adv = adv_store[:N * T].view(N, T)
            ret = ret_store[:N * T].view(N, T)
            rl.gae(dev["rewards"], dev["values"], flags["terminated"], flags["truncated"],
                   dev["trunc_values"], dev["bootstrap"], 0.99, 0.95, advantages=adv,
                   returns=ret)
            what = f"round {rnd} {N}x{T} {dtype}"
            check(adv, oa, dtype, f"gae {what}")
            check(ret, orr, dtype, f"gae returns {what}")
            tr = rl.eligibility_traces(x, flags["terminated"], rl.RESET_AFTER_DONE, 0.99, 0.9,
                                       out=adv)
            check(tr, ot, dtype, f"traces {what}")
