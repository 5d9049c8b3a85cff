"""Calls on the caller's streams: the library enqueues on the stream it is
given (the binding passes the current one) and keeps no state between
calls, so calls on two streams may run at the same time.  Two streams of
default priority each get a single call, a batch and a fused consumer call;
every output must equal, bit for bit, the same call made alone on the
default stream.  Then four host threads, each on a stream of its own, make
such calls at the same time (ctypes releases the interpreter lock during
each C call, so the library is entered from several threads at once)."""
import threading

import numpy as np
import pytest
import torch

import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def inputs(seed, N, T):
    d = workloads.backward_rollout(seed, N, T, p_term=0.02, p_trunc=0.02)
    f = workloads.forward_rollout(seed + 1, N, T, p_start=0.02)
    return d, f


def work(d, f):
    """Each call's outputs, enqueued on the current stream."""
    out = []
    out += list(rl.gae(dev(d.rewards), dev(d.values), dev(d.terminated), dev(d.truncated),
                       dev(d.trunc_values), dev(d.bootstrap), 0.99, 0.95))
    b = rl.Batch()
    out.append(b.td_lambda(dev(d.rewards), dev(d.values), dev(d.terminated), None, None,
                           dev(d.bootstrap), 0.97, 0.9))
    out.append(b.eligibility_traces(dev(f.increments), dev(f.starts), rl.RESET_ON_START,
                                    0.99, 0.9))
    out.append(b.episodic_prefix_sum(dev(f.ints), dev(f.starts), rl.RESET_ON_START))
    b.run()
    adv, ret, stats = rl.gae_stats(dev(d.rewards), dev(d.values), dev(d.terminated))
    out += [adv, ret, stats]
    return out


def test_calls_on_two_streams(gpu_device):
    cases = [inputs(11, 3000, 256), inputs(21, 700, 1000)]
    alone = []
    for d, f in cases:
        alone.append(work(d, f))
        torch.cuda.synchronize(gpu_device)
    streams = [torch.cuda.Stream(device=gpu_device), torch.cuda.Stream(device=gpu_device)]
    got = []
    for rep in range(3):
        outs = []
        for (d, f), s in zip(cases, streams):
            with torch.cuda.stream(s):
                outs.append(work(d, f))
        torch.cuda.synchronize(gpu_device)
        got.append(outs)
    for rep, outs in enumerate(got):
        for k, (o, a) in enumerate(zip(outs, alone)):
            for j, (x, y) in enumerate(zip(o, a)):
                assert torch.equal(x, y), f"repeat {rep}, stream {k}, output {j} differs"


def test_calls_from_host_threads(gpu_device):
    cases = [inputs(31 + 10 * k, 1000 + 500 * k, 128 * (k + 1)) for k in range(4)]
    alone = []
    for d, f in cases:
        alone.append(work(d, f))
        torch.cuda.synchronize(gpu_device)
    results = [None] * len(cases)
    errors = []
    start = threading.Barrier(len(cases))

    def run(k):
        try:
            torch.cuda.set_device(gpu_device)
            s = torch.cuda.Stream(device=gpu_device)
            start.wait(timeout=60)
            with torch.cuda.stream(s):
                outs = [work(*cases[k]) for _ in range(5)]
            s.synchronize()
            results[k] = outs
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {k}: {e!r}")

    threads = [threading.Thread(target=run, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for k, outs in enumerate(results):
        for rep, o in enumerate(outs):
            for j, (x, y) in enumerate(zip(o, alone[k])):
                assert torch.equal(x, y), f"thread {k}, repeat {rep}, output {j} differs"
