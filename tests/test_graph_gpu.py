"""The library's calls under HIP graph capture: a batch (grouped and single
launches, fp32 and bf16), a chunked call and the fused PPO consumers,
captured once and replayed several times with the program's own eager work
and synchronizations between replays.  Every replay must equal the eager
result bit for bit (the library records no memset and allocates nothing,
so a captured call is the same kernels on the same buffers)."""
import numpy as np
import pytest
import torch

import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu


def dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_graph_replays_equal_eager(gpu_device):
    d = workloads.backward_rollout(11, 512, 128, p_term=0.05, p_trunc=0.05)
    r, v, t, tr, tv, b = (dev(x) for x in (d.rewards, d.values, d.terminated, d.truncated,
                                           d.trunc_values, d.bootstrap))
    mu, pi = dev(d.behaviour_logp), dev(d.target_logp)
    long = workloads.backward_rollout(12, 3, 20000)
    lr, lv, lt = dev(long.rewards), dev(long.values), dev(long.terminated)
    f = workloads.forward_rollout(13, 64, 512)
    x, st = dev(f.increments), dev(f.starts)

    # outputs and workspaces allocated before capture (the library allocates nothing)
    outs = {k: torch.empty(512, 128, device=gpu_device) for k in ("adv", "ret", "td", "vs", "pg",
                                                                     "adv2", "ret2", "grad")}
    outs["traces"] = torch.empty(64, 512, device=gpu_device)
    outs["long"] = torch.empty(3, 20000, device=gpu_device)
    outs["bf"] = torch.empty(512, 128, dtype=torch.bfloat16, device=gpu_device)
    stats = torch.empty(2, dtype=torch.float64, device=gpu_device)
    loss = torch.empty(1, dtype=torch.float64, device=gpu_device)
    rb, vb = r.bfloat16(), v.bfloat16()

    batch = rl.Batch()
    batch.gae(r, v, t, tr, tv, b, advantages=outs["adv"], returns=outs["ret"])
    batch.td_lambda(r, v, t, tr, tv, b, out=outs["td"])
    batch.vtrace(r, v, mu, pi, t, vs=outs["vs"], pg_advantages=outs["pg"])
    batch.eligibility_traces(x, st, out=outs["traces"])          # one-wave class
    batch.td_lambda(rb, vb, t, out=outs["bf"])                    # bf16 group
    batch.gae(lr, lv, lt, advantages=outs["long"], with_returns=False)   # chunked

    def step():
        batch.run()
        rl.gae_stats(r, v, t, tr, tv, b, advantages=outs["adv2"], returns=outs["ret2"],
                     stats=stats)
        rl.ppo_clip_loss(outs["adv2"], pi, mu, stats, grad=outs["grad"])

    # the fused calls allocate their workspace and loss through torch: warm the
    # caching allocator on a side stream first, as torch requires for capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = {k: o.clone() for k, o in outs.items()}
    eager_stats = stats.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for o in outs.values():
            o.fill_(float("nan"))
        stats.fill_(float("nan"))
        # unrelated eager work and a synchronize between replays
        torch.cumsum(torch.randn(1 << 16, device=gpu_device), 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, o in outs.items():
            assert torch.equal(o, eager[k]), f"replay {rep}: {k} differs from eager"
        assert torch.equal(stats, eager_stats), f"replay {rep}: stats differ"
