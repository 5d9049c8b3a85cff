"""The largest calls: more than 2^31 env-steps in one call, so that every flat
index passes 32 bits, on each launch shape (rows spanning waves, wave-local
rows, one-wave row walks, skewed windows, all in grids of more than 2^20
workgroups, and 512 rows of 2^22 + 4 steps walked by 16-wave workgroups);
2^31 rows of one step, the most rows the ABI takes; and rows of
2^30 steps, the longest, on the chunked path (1.5 million chunks).

Inputs are drawn on the device (workloads.device_rollout, seeded).  Outputs
are checked against the fp64 oracle on samples whose values they determine
alone, at the parity bar 1e-4 * (1 + |oracle|) (bit-exact for int32):
  * whole rows, since rows are independent: the first two, the last two and
    28 random ones;
  * in rows of 2^30 steps, whole episode segments: a backward segment starts
    after a terminated step and ends at the next one (or at the row end, with
    the row's bootstrap), a forward one runs from a start flag to the next
    (or to the row end), and nothing outside a segment reaches its outputs.
Each case needs up to about 75 GB of device memory and frees it after."""
import numpy as np
import pytest
import torch

import oracle
import linear_recurrence_scan_row_amd as rl
from linear_recurrence_scan_row_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-4
G, LAM, TLAM = 0.99, 0.95, 0.9
BACKWARD = ("rewards", "values", "trunc_values", "terminated", "truncated", "bootstrap")


def f32(x):
    return float(np.float32(x))


def close(gpu, ref, what):
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ref, np.float64)
    assert g.shape == o.shape, what
    err = np.abs(g - o) / (1.0 + np.abs(o))
    assert err.max() <= TOL, f"{what}: max scaled error {err.max():.3e}"


def sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, N - 2, N - 1], rng.integers(0, N, 28)]))


def take(x, rows):
    """The sampled rows (or entries of a per-row array) as host arrays."""
    idx = torch.from_numpy(rows).to(x.device)
    return x.index_select(0, idx).cpu().numpy()


@pytest.fixture
def fresh(gpu_device):
    if torch.cuda.get_device_properties(gpu_device).total_memory < 100 << 30:
        pytest.skip("needs about 75 GB of device memory")
    torch.cuda.empty_cache()
    yield gpu_device
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


SHAPES = [
    pytest.param(2**21 + 3, 1024, id="rows spanning waves"),
    pytest.param(2**24 + 5, 128, id="wave-local rows"),
    pytest.param(2**22 + 1, 512, id="one-wave row walks"),
    pytest.param(2**21 + 4099, 1023, id="skewed windows"),
    pytest.param(512, 2**22 + 4, id="16-wave row walks"),
]


@pytest.mark.parametrize("N,T", SHAPES)
def test_gae_past_32_bit_indices(N, T, fresh):
    assert N * T > 2**31
    d = workloads.device_rollout(N + T, N, T, fresh, BACKWARD)
    adv, ret = rl.gae(d["rewards"], d["values"], d["terminated"], d["truncated"],
                      d["trunc_values"], d["bootstrap"], G, LAM)
    rows = sample_rows(N, N + T)
    h = {k: take(v, rows) for k, v in d.items()}
    oa, orr = oracle.gae(h["rewards"], h["values"], h["terminated"], h["truncated"],
                         h["trunc_values"], h["bootstrap"], f32(G), f32(LAM))
    close(take(adv, rows), oa, f"gae {N}x{T}")
    close(take(ret, rows), orr, f"gae returns {N}x{T}")


@pytest.mark.parametrize("N,T", SHAPES)
def test_forward_scans_past_32_bit_indices(N, T, fresh):
    d = workloads.device_rollout(N * 3 + T, N, T, fresh, ("increments", "ints", "starts"))
    rows = sample_rows(N, N * 3 + T)
    e = rl.eligibility_traces(d["increments"], d["starts"], rl.RESET_ON_START, G, TLAM)
    x, st = take(d["increments"], rows), take(d["starts"], rows)
    close(take(e, rows), oracle.eligibility_traces(x, st, oracle.RESET_ON_START, f32(G),
                                                   f32(TLAM)), f"traces {N}x{T}")
    del e
    s = rl.episodic_prefix_sum(d["ints"], d["starts"], rl.RESET_ON_START)
    want = oracle.episodic_prefix_sum(take(d["ints"], rows), st, oracle.RESET_ON_START)
    assert np.array_equal(take(s, rows), want), f"int32 prefix sum {N}x{T}"


def test_most_rows(fresh):
    """2^31 rows of one step: every step is its row's end."""
    N, T = 2**31, 1
    d = workloads.device_rollout(31, N, T, fresh, ("rewards", "terminated", "bootstrap"),
                                 p_term=0.3)
    out = rl.discounted_returns(d["rewards"], d["terminated"], bootstrap=d["bootstrap"],
                                gamma=G)
    rows = sample_rows(N, 31)
    h = {k: take(v, rows) for k, v in d.items()}
    close(take(out, rows), oracle.discounted_returns(h["rewards"], h["terminated"], None, None,
                                                     h["bootstrap"], f32(G)),
          "discounted returns 2^31 x 1")


def _segments(flags_row, T, seed, backward, k=12):
    """[a, e) step ranges of whole episode segments of one row (flags on the
    device): the first, the last and k random ones."""
    pos = torch.nonzero(flags_row).flatten().cpu().numpy()
    assert pos.size > k + 2, "too few episode boundaries for the sample"
    if backward:   # a terminated step ends its segment
        bounds = np.concatenate([[-1], pos, [T - 1]])
        segs = [(bounds[j] + 1, bounds[j + 1] + 1) for j in range(bounds.size - 1)]
    else:          # a start flag begins one
        bounds = np.concatenate([[0], pos, [T]])
        segs = [(bounds[j], bounds[j + 1]) for j in range(bounds.size - 1)]
    segs = [(a, e) for a, e in segs if e > a]
    rng = np.random.default_rng(seed)
    pick = rng.choice(len(segs) - 2, size=k, replace=False) + 1
    return [segs[0], segs[-1]] + [segs[j] for j in sorted(pick)]


def test_longest_rows_chunked(fresh):
    """Three rows of 2^30 steps: the chunked path, 2^19 chunks per row, one
    workgroup per chunk in grids of 1.5 million workgroups."""
    N, T = 3, 2**30
    d = workloads.device_rollout(30, N, T, fresh, BACKWARD)
    adv, ret = rl.gae(d["rewards"], d["values"], d["terminated"], d["truncated"],
                      d["trunc_values"], d["bootstrap"], G, LAM)
    boot = d["bootstrap"].cpu().numpy()
    for row in range(N):
        for a, e in _segments(d["terminated"][row], T, 30 + row, backward=True):
            h = {k: d[k][row, a:e].cpu().numpy()[None] for k in
                 ("rewards", "values", "terminated", "truncated", "trunc_values")}
            oa, orr = oracle.gae(h["rewards"], h["values"], h["terminated"], h["truncated"],
                                 h["trunc_values"], boot[row:row + 1], f32(G), f32(LAM))
            close(adv[row, a:e].cpu().numpy()[None], oa, f"gae row {row} steps {a}..{e}")
            close(ret[row, a:e].cpu().numpy()[None], orr, f"gae returns row {row} steps {a}..{e}")
    del adv, ret, d
    torch.cuda.empty_cache()
    f = workloads.device_rollout(32, N, T, fresh, ("increments", "starts"))
    tr = rl.eligibility_traces(f["increments"], f["starts"], rl.RESET_ON_START, G, TLAM)
    for row in range(N):
        for a, e in _segments(f["starts"][row], T, 32 + row, backward=False):
            x = f["increments"][row, a:e].cpu().numpy()[None]
            st = f["starts"][row, a:e].cpu().numpy()[None]
            close(tr[row, a:e].cpu().numpy()[None],
                  oracle.eligibility_traces(x, st, oracle.RESET_ON_START, f32(G), f32(TLAM)),
                  f"traces row {row} steps {a}..{e}")
