"""The benchmark's timed steps, checked against the fp64 oracle at full size.

bench.py times each workload as one rlca_run_batch holding the step's calls:
the four GAE / TD(lambda) calls over 4096 x 128 and the four forward-workload
calls over 16384 x 512 share one grouped launch each, and a one-call step
(V-Trace 4096 x 256, Retrace 2048 x 1024, GAE 8 x 16) runs the call's own
kernel, and the few-long-rows steps (8 x 131072, 1 x 2^20) run each call's
three chunked launches.  These tests build those batches with bench.py's own call tables,
rotation sets and recording code, run one step and compare every output of
every call with the oracle on the same inputs:

  * fp32 storage: |gpu - oracle| <= 1e-4 * (1 + |oracle|), int32 bit-exact;
  * bf16 / fp16 storage: the oracle runs on the inputs as the kernel sees
    them (rounded to the storage type, widened exactly), and the bar adds the
    one rounding of each stored output, |g - o| <= 1e-4 * (1 + |o|) * (1 + u)
    + u * |o| with unit roundoff u = 2^-8 (bf16) or 2^-11 (fp16).
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from linear_recurrence_scan_row_amd import rlca, workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
REAL = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
UNIT_ROUNDOFF = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def _seen_by_kernel(arrays, dtype):
    """Host inputs as the kernel reads them: real arrays rounded to the
    storage type and widened back exactly; flags and int32 unchanged."""
    out = {}
    for k, v in arrays.items():
        if v.dtype == np.float32 and dtype != "f32":
            v = torch.from_numpy(np.ascontiguousarray(v)).to(REAL[dtype]).float().numpy()
        out[k] = v
    return out


def _oracle(call_name, h, cfg):
    """The oracle's outputs for one call of a bench step, in call order, with
    the parameters as the library receives them (fp32)."""
    g = float(np.float32(cfg["gamma"]))
    lam = float(np.float32(cfg.get("lam", 0.95)))
    if call_name in ("gae", "gae+trunc", "td_lambda", "td_lambda+trunc"):
        tr = call_name.endswith("+trunc")
        args = (h["r"], h["v"], h["term"], h["trunc"] if tr else None, h["tv"] if tr else None,
                h["b"], g, lam)
        if call_name.startswith("gae"):
            return oracle.gae(*args)
        return (oracle.td_lambda(*args),)
    if call_name == "vtrace":
        return oracle.vtrace(h["r"], h["v"], h["mu"], h["pi"], h["term"], None, None, h["b"],
                             g, lam, cfg["rho_bar"], cfg["c_bar"])
    if call_name == "retrace+trunc":
        return (oracle.retrace(h["r"], h["q"], h["eq"], h["mu"], h["pi"], h["term"], h["trunc"],
                               h["tv"], h["b"], g, lam, cfg["c_bar"]),)
    if call_name == "discounted":
        return (oracle.discounted_returns(h["r"], h["dones"], None, None, h["b"], g),)
    if call_name == "eligibility" and "x" not in h:
        # the few-long-rows steps: traces over the rewards, resets after
        # terminated steps
        return (oracle.eligibility_traces(h["r"], h["term"], oracle.RESET_AFTER_DONE, g, lam),)
    if call_name == "eligibility":
        return (oracle.eligibility_traces(h["x"], h["starts"], oracle.RESET_ON_START, g, lam),)
    if call_name == "prefix_sum_f32":
        return (oracle.episodic_prefix_sum(h["r"], h["starts"], oracle.RESET_ON_START),)
    if call_name == "prefix_sum_i32":
        return (oracle.episodic_prefix_sum(h["xi"], h["starts"], oracle.RESET_ON_START),)
    raise AssertionError(f"no oracle for {call_name}")


def _check(gpu, ref, dtype, what):
    if gpu.dtype == torch.int32:
        g = gpu.cpu().numpy()
        assert np.array_equal(g, ref), f"{what}: {np.count_nonzero(g != ref)} int32 mismatches"
        return
    g = gpu.float().cpu().numpy().astype(np.float64)
    o = np.asarray(ref, np.float64)
    assert g.shape == o.shape, what
    u = UNIT_ROUNDOFF[dtype]
    bound = TOL * (1 + np.abs(o)) * (1 + u) + u * np.abs(o)
    excess = np.abs(g - o) - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[worst] <= 0, (f"{what}: |gpu - oracle| = {abs(g[worst] - o[worst]):.3e} > "
                                f"{bound[worst]:.3e} at {worst}: gpu {g[worst]!r} "
                                f"oracle {o[worst]!r}")


STEPS = [("gae_td_4096x128", "f32"), ("gae_td_4096x128", "bf16"), ("gae_td_4096x128", "f16"),
         ("vtrace_4096x256", "f32"), ("vtrace_4096x256", "bf16"),
         ("retrace_2048x1024", "f32"), ("retrace_2048x1024", "bf16"),
         ("forward_16384x512", "f32"), ("forward_16384x512", "bf16"),
         ("gae_8x16", "f32"), ("long_8x131072", "f32"), ("long_1x1048576", "f32")]


@pytest.mark.parametrize("name,dtype", STEPS)
def test_bench_step_matches_oracle(name, dtype, gpu_device, monkeypatch):
    cfg = dict(workloads.CONFIGS[name])
    host = workloads.make(name)
    real = REAL[dtype]
    arrays, calls = bench.workload_calls(name, cfg, host, real.itemsize)
    ncalls = len(calls)
    # one rotation set per call, as in the bench's first step
    monkeypatch.setattr(bench, "COLD_BYTES", (ncalls - 1) * min(c[3] for c in calls))
    sets = bench.make_sets(torch, arrays, calls, gpu_device, min(c[3] for c in calls), real)
    assert len(sets) >= ncalls
    for s in sets[:ncalls]:
        for k in ("o0", "o1"):
            s[k].fill_(float("nan"))
        s["oi"].fill_(-1)
    storage = bench.STORAGE[dtype]
    recorded = [bench.batch_record(rlca, calls[c], sets[c], storage) for c in range(ncalls)]
    stream = torch.cuda.current_stream(gpu_device)
    fn, args = bench.bind_batch(rlca.lib(), rlca, recorded, stream.cuda_stream)
    st = fn(*args)
    assert st == 0, f"{name} {dtype}: rlca_run_batch returned {rlca.STATUS_NAMES.get(st, st)}"
    torch.cuda.synchronize(gpu_device)

    h = _seen_by_kernel(arrays, dtype)
    for c, call in enumerate(calls):
        refs = _oracle(call[0], h, cfg)
        outs = call[4]
        assert len(outs) == len(refs), call[0]
        for key, ref in zip(outs, refs):
            _check(sets[c][key], ref, dtype, f"{name} {dtype} {call[0]} {key}")
