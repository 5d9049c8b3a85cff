#!/usr/bin/env python3
"""Throughput benchmark of the fused credit-assignment scans on one MI355X.

Default workload: GAE and TD(lambda) returns over 4096 envs x 128 steps, fp32,
each with and without per-step truncation handling; one *step* is those four
library calls over one rollout (inputs resident in HBM).  Prints ONE JSON line.

Measurement:
  * cold cache: every call reads a different copy of the rollout, rotating
    over >= 1 GiB of copies, so neither the 4 MB-per-XCD L2 nor the 256 MB
    Infinity Cache can serve the operands (the fused consumers' small
    workspaces are one per consumer, as a caller keeps them);
  * each step is one rlca_run_batch holding the step's calls, which share one
    grouped launch (pre-bound ctypes call, asynchronous on one stream);
    --launch eager makes one library call per estimator instead, and
    --launch graph captures those calls into a HIP graph per step and replays
    it;
  * whole-step time: HIP events around K steps, synchronised on both sides;
    per-kernel time: HIP events around back-to-back launches of one call
    variant (rotating sets), averaged; with --launch batch the roofline is
    that of the grouped launch over the whole step's bytes;
  * full_call_us: the pages' protocol per call (20 untimed calls, 5 trials
    of 50 calls each between its own events and followed by a synchronize;
    minimum of the trial medians), host launch included;
  * effective GB/s uses the algorithmic byte model: every input array read
    once and every output written once at dense size (fp32 / int32 4 B, bf16
    / fp16 2 B, flags 1 B per step, bootstrap one value per row);
  * copy_ceiling: a torch device copy moving the step's bytes, cold and back
    to back, as the attainable ceiling at this size;
  * floor: bench_floor.hip moving exactly the step's bytes with the
    library's tiling and access widths and no arithmetic (one launch per
    step, same rotation); value_over_floor = floor time / step time;
  * roofline: the dominant kernel's average duration from the committed
    rocprofv3 kernel-trace summary (profiles/kernels_<workload>.md) when it
    was taken on the current kernel sources, else from the events; the
    event-timed figures are kept beside it (*_event); roofline_gae_call is
    the GAE call's own kernel, the one the metric names;
  * cpu_baseline: the fp64 sequential oracle on this host, single thread;
    cpu_baseline_all_cores: the same with the rows split over up to 16
    worker processes; host_cores: the CPUs this process may run on
    (affinity), nproc and os.cpu_count().

Workloads: the five configurations (gae_8x16, gae_td_4096x128,
vtrace_4096x256, retrace_2048x1024, forward_16384x512), the fused PPO
consumers (ppo_4096x128) and few long rows on the chunked path
(long_1x1048576, long_8x131072: GAE with truncation and eligibility traces).

--sweep [sizes|long] prints one JSON line per (num_envs, T, estimator) of a
size sweep instead (three trials per point, the fastest kept): rollout shapes,
or few long rows on both sides of the chunked path's row threshold.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E peak, 8 TB/s
METRIC = "effective HBM GB/s (% of peak) + env-steps/s, GAE 4096×128 fp32"
COLD_BYTES = 1 << 30
WORKSPACE_BYTES = 1 << 20   # per workspace buffer of the fused consumers


# ------------------------------------------------------------------ workloads
# A call: (name, library function, argument template, bytes per launch).
# Argument templates name buffers of a rotation set ("@key") or give scalars.


def _backward_bytes(nt, n, real_in, flags, real_out, es=4):
    return nt * (es * real_in + flags + es * real_out) + es * n


# --dtype: storage type of the real-valued arrays (rlca_dtype codes)
STORAGE = {"f32": 0, "bf16": 2, "f16": 3}


def workload_calls(name, cfg, host, es=4):
    """Return (arrays, calls) for a named workload; arrays are the host inputs
    each rotation set holds, calls the per-step library calls.  `es` is the
    byte size of a stored real value."""
    n, t = host.num_envs, host.T
    nt = n * t
    g = cfg["gamma"]
    lam = cfg.get("lam", 0.95)
    if name in ("gae_td_4096x128", "gae_8x16"):
        arrays = dict(r=host.rewards, v=host.values, term=host.terminated,
                      trunc=host.truncated, tv=host.trunc_values, b=host.bootstrap)
        gae_nt = ("gae", "rlca_gae",
                  ["@r", "@v", "@term", None, None, "@b", g, lam, n, t, "@o0", "@o1"],
                  _backward_bytes(nt, n, 2, 1, 2, es), ("o0", "o1"))
        gae_tr = ("gae+trunc", "rlca_gae",
                  ["@r", "@v", "@term", "@trunc", "@tv", "@b", g, lam, n, t, "@o0", "@o1"],
                  _backward_bytes(nt, n, 3, 2, 2, es), ("o0", "o1"))
        td_nt = ("td_lambda", "rlca_td_lambda",
                 ["@r", "@v", "@term", None, None, "@b", g, lam, n, t, "@o0"],
                 _backward_bytes(nt, n, 2, 1, 1, es), ("o0",))
        td_tr = ("td_lambda+trunc", "rlca_td_lambda",
                 ["@r", "@v", "@term", "@trunc", "@tv", "@b", g, lam, n, t, "@o0"],
                 _backward_bytes(nt, n, 3, 2, 1, es), ("o0",))
        calls = [gae_tr] if name == "gae_8x16" else [gae_nt, gae_tr, td_nt, td_tr]
        return arrays, calls
    if name.startswith("long_"):
        # few long rows: GAE with truncation, and eligibility traces over the
        # rewards with resets after terminated steps
        arrays = dict(r=host.rewards, v=host.values, term=host.terminated,
                      trunc=host.truncated, tv=host.trunc_values, b=host.bootstrap)
        calls = [
            ("gae+trunc", "rlca_gae",
             ["@r", "@v", "@term", "@trunc", "@tv", "@b", g, lam, n, t, "@o0", "@o1"],
             _backward_bytes(nt, n, 3, 2, 2, es), ("o0", "o1")),
            ("eligibility", "rlca_eligibility_traces",
             ["@r", "@term", 1, g, lam, n, t, "@o0"], nt * (2 * es + 1), ("o0",)),
        ]
        return arrays, calls
    if name == "ppo_4096x128":
        # the fused consumers: GAE + advantage statistics, then the PPO loss
        # and its gradient with on-the-fly normalization
        arrays = dict(r=host.rewards, v=host.values, term=host.terminated,
                      trunc=host.truncated, tv=host.trunc_values, b=host.bootstrap,
                      mu=host.behaviour_logp, pi=host.target_logp)
        calls = [
            ("gae_stats", "rlca_gae_stats",
             ["@r", "@v", "@term", "@trunc", "@tv", "@b", g, lam, n, t, "@o0", "@o1", "@stats",
              "@ws", WORKSPACE_BYTES],
             _backward_bytes(nt, n, 3, 2, 2) + 16, ("o0", "o1")),
            ("ppo_clip_loss", "rlca_ppo_clip_loss",
             ["@o0", "@stats", "@pi", "@mu", cfg["clip_eps"], 1e-8, n, t, "@grad", "@loss",
              "@ws2", WORKSPACE_BYTES],
             nt * 16 + 16 + 8, ("grad",)),
        ]
        return arrays, calls
    if name == "vtrace_4096x256":
        arrays = dict(r=host.rewards, v=host.values, mu=host.behaviour_logp,
                      pi=host.target_logp, term=host.terminated, b=host.bootstrap)
        call = ("vtrace", "rlca_vtrace",
                ["@r", "@v", "@mu", "@pi", "@term", None, None, "@b", g, lam, cfg["rho_bar"],
                 cfg["c_bar"], n, t, "@o0", "@o1"],
                _backward_bytes(nt, n, 4, 1, 2, es), ("o0", "o1"))
        return arrays, [call]
    if name == "retrace_2048x1024":
        arrays = dict(r=host.rewards, q=host.q_values, eq=host.expected_q,
                      mu=host.behaviour_logp, pi=host.target_logp, term=host.terminated,
                      trunc=host.truncated, tv=host.trunc_values, b=host.bootstrap)
        call = ("retrace+trunc", "rlca_retrace",
                ["@r", "@q", "@eq", "@mu", "@pi", "@term", "@trunc", "@tv", "@b", g, lam,
                 cfg["c_bar"], n, t, "@o0"],
                _backward_bytes(nt, n, 6, 2, 1, es), ("o0",))
        return arrays, [call]
    if name == "forward_16384x512":
        arrays = dict(r=host.rewards, x=host.increments, xi=host.ints, starts=host.starts,
                      dones=host.dones, b=host.bootstrap)
        calls = [
            ("discounted", "rlca_discounted_returns",
             ["@r", "@dones", None, None, "@b", g, n, t, "@o0"],
             _backward_bytes(nt, n, 1, 1, 1, es), ("o0",)),
            ("eligibility", "rlca_eligibility_traces",
             ["@x", "@starts", 0, g, lam, n, t, "@o0"], nt * (2 * es + 1), ("o0",)),
            ("prefix_sum_f32", "rlca_episodic_prefix_sum",
             ["@r", 0, "@starts", 0, n, t, "@o0"], nt * (2 * es + 1), ("o0",)),
            ("prefix_sum_i32", "rlca_episodic_prefix_sum",
             ["@xi", 1, "@starts", 0, n, t, "@oi"], nt * 9, ("oi",)),
        ]
        return arrays, calls
    raise SystemExit(f"unknown workload {name}")


# ------------------------------------------------------------------ GPU timing


def make_sets(torch, arrays, calls, device, min_call_bytes, real=None):
    """Rotation sets: full copies of the inputs plus every output buffer, as
    many as needed for >= COLD_BYTES of traffic between reuses of a set.
    Real-valued arrays are stored as `real` (a torch dtype; float32 if None)."""
    real = real or torch.float32
    master = {}
    for k, v in arrays.items():
        x = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        master[k] = x.to(real) if x.dtype == torch.float32 else x
    shape = next(v.shape for v in arrays.values() if v.ndim == 2)
    nsets = min(4096, max(2, -(-COLD_BYTES // max(1, min_call_bytes)) + 1))
    per_set = sum(v.numel() * v.element_size() for v in master.values()) + \
        sum(4 * int(np.prod(shape)) for _ in range(3))
    nsets = int(min(nsets, max(2, (24 << 30) // per_set)))
    sets = []
    named = {a[1:] for c in calls for a in c[2] if isinstance(a, str) and a.startswith("@")}
    for _ in range(nsets):
        s = {k: v.clone() for k, v in master.items()}
        s["o0"] = torch.zeros(shape, dtype=real, device=device)
        s["o1"] = torch.zeros(shape, dtype=real, device=device)
        s["oi"] = torch.empty(shape, dtype=torch.int32, device=device)
        if "grad" in named:
            s["grad"] = torch.empty(shape, dtype=torch.float32, device=device)
        for k in ("stats", "loss"):
            if k in named:
                s[k] = torch.zeros(2, dtype=torch.float64, device=device)
        sets.append(s)
    # the fused consumers' workspaces (ticket counters and per-workgroup
    # partial sums, zero-filled once; every call leaves them so) are one per
    # consumer for the whole rotation, as a caller keeps one per stream: the
    # rotation keeps the inputs and outputs cold, not the library's state
    for k in ("ws", "ws2"):
        if k in named:
            ws = torch.zeros(WORKSPACE_BYTES, dtype=torch.uint8, device=device)
            for s in sets:
                s[k] = ws
    return sets


# Positional arguments of each entry point, named as the rlca_call fields they
# fill when the same call is recorded into a batch.
_BACKWARD_HEAD = ["rewards", "values", "terminated", "truncated", "trunc_values", "bootstrap",
                  "gamma", "lambda_", "num_envs", "T"]
BATCH_FIELDS = {
    "rlca_gae": (0, _BACKWARD_HEAD + ["out0", "out1"]),
    "rlca_td_lambda": (1, _BACKWARD_HEAD + ["out0"]),
    "rlca_discounted_returns": (2, ["rewards", "terminated", "truncated", "trunc_values",
                                    "bootstrap", "gamma", "num_envs", "T", "out0"]),
    "rlca_vtrace": (3, ["rewards", "values", "behaviour_logp", "target_logp", "terminated",
                        "truncated", "trunc_values", "bootstrap", "gamma", "lambda_",
                        "rho_bar", "c_bar", "num_envs", "T", "out0", "out1"]),
    "rlca_retrace": (4, ["rewards", "values", "expected_q", "behaviour_logp", "target_logp",
                         "terminated", "truncated", "trunc_values", "bootstrap", "gamma",
                         "lambda_", "c_bar", "num_envs", "T", "out0"]),
    "rlca_eligibility_traces": (5, ["rewards", "terminated", "convention", "gamma", "lambda_",
                                    "num_envs", "T", "out0"]),
    "rlca_episodic_prefix_sum": (6, ["rewards", "dtype", "terminated", "convention",
                                     "num_envs", "T", "out0"]),
}


# ------------------------------------------------------------------ streaming floor
# bench_floor.hip moves exactly a step's bytes with the library's tiling and
# access widths and does no arithmetic; one launch per step covers every call.
FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")
_PER_STEP_IN = {"rewards", "values", "expected_q", "behaviour_logp", "target_logp",
                "terminated", "truncated", "trunc_values"}


def _roles(names):
    return ["in" if f in _PER_STEP_IN else "row" if f == "bootstrap" else
            "out" if f in ("out0", "out1") else None for f in names]


FLOOR_ROLES = {fname: _roles(names) for fname, (_, names) in BATCH_FIELDS.items()}
FLOOR_ROLES["rlca_gae_stats"] = FLOOR_ROLES["rlca_gae"] + [None, None, None]
FLOOR_ROLES["rlca_ppo_clip_loss"] = ["in", None, "in", "in", None, None, None, None, "out",
                                     None, None, None]


class _FloorCall(ctypes.Structure):
    # inputs ordered by element size: n4 4-byte, then n2 2-byte, then n1 1-byte;
    # magic, shift and sig are filled in by bench_floor_launch
    _fields_ = [("ins", ctypes.c_void_p * 9), ("outs", ctypes.c_void_p * 2),
                ("row", ctypes.c_void_p), ("steps", ctypes.c_uint64), ("T", ctypes.c_uint32),
                ("tiles", ctypes.c_uint32), ("magic", ctypes.c_uint32),
                ("shift", ctypes.c_uint32), ("n4", ctypes.c_uint8), ("n2", ctypes.c_uint8),
                ("n1", ctypes.c_uint8), ("nout", ctypes.c_uint8), ("out_bytes", ctypes.c_uint8),
                ("row_bytes", ctypes.c_uint8), ("sig", ctypes.c_uint8), ("pad", ctypes.c_uint8)]


class _FloorLaunch(ctypes.Structure):
    _fields_ = [("calls", _FloorCall * 8), ("ncalls", ctypes.c_uint32)]


def floor_record(calls, bufs_per_call, n, t):
    """The floor launch moving the bytes of one step: calls[c] on bufs_per_call[c]."""
    rec = _FloorLaunch()
    rec.ncalls = len(calls)
    for c, (call, bufs) in enumerate(zip(calls, bufs_per_call)):
        _, fname, template, _, _ = call
        f = rec.calls[c]
        ins, outs = [], []
        for role, a in zip(FLOOR_ROLES[fname], template):
            if role is None or not (isinstance(a, str) and a.startswith("@")):
                continue
            x = bufs[a[1:]]
            if role == "in":
                ins.append((x.element_size(), x.data_ptr()))
            elif role == "out":
                outs.append((x.element_size(), x.data_ptr()))
            else:
                f.row, f.row_bytes = x.data_ptr(), x.element_size()
        ins.sort(key=lambda e: -e[0])   # stable: 4-byte, then 2-byte, then 1-byte streams
        for k, (_, ptr) in enumerate(ins):
            f.ins[k] = ptr
        f.n4, f.n2, f.n1 = (sum(1 for e, _ in ins if e == w) for w in (4, 2, 1))
        if len({e for e, _ in outs}) != 1 or f.n4 + f.n2 + f.n1 != len(ins):
            raise ValueError(f"{fname}: streams the floor kernel does not take")
        for k, (_, ptr) in enumerate(outs):
            f.outs[k] = ptr
        f.nout, f.out_bytes = len(outs), outs[0][0]
        f.steps, f.T = n * t, t
        f.tiles = (n * t + 2047) // 2048
    return rec


def _resolve(a, bufs):
    return bufs[a[1:]].data_ptr() if isinstance(a, str) and a.startswith("@") else a


def batch_record(rlca, call, bufs, storage=0):
    """The rlca_call that records `call` on rotation set `bufs`, its real
    arrays stored as `storage` (an rlca_dtype; int32 sums keep RLCA_I32)."""
    _, fname, template, _, _ = call
    op, names = BATCH_FIELDS[fname]
    c = rlca.RlcaCall(op=op)
    for name, a in zip(names, template):
        setattr(c, name, _resolve(a, bufs))
    if c.dtype != rlca.RLCA_I32:
        c.dtype = storage
    return c


def bind_batch(lib, rlca, recorded, stream):
    arr = (rlca.RlcaCall * len(recorded))(*recorded)
    return lib.rlca_run_batch, (arr, len(recorded), stream)


def bind(lib, call, bufs, stream):
    _, fname, template, _, _ = call
    return getattr(lib, fname), tuple(_resolve(a, bufs) for a in template) + (stream,)


def run_gpu(args, name, cfg, host):
    import torch
    from linear_recurrence_scan_row_amd import rlca

    lib = rlca.lib()
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    storage = STORAGE[args.dtype]
    if any(c[1] not in BATCH_FIELDS for c in workload_calls(name, cfg, host)[1]):
        if args.dtype != "f32":
            raise SystemExit(f"{name} runs in fp32 only")
        args.launch = "eager"   # calls that rlca_run_batch does not take
    real = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.dtype]
    arrays, calls = workload_calls(name, cfg, host, real.itemsize)
    sets = make_sets(torch, arrays, calls, device, min(c[3] for c in calls), real)

    def bind_call(call, bufs, h):
        # bf16 / fp16 calls go through rlca_run_batch (the single-call entry
        # points other than the prefix sum are fp32)
        if storage == 0:
            return bind(lib, call, bufs, h)
        return bind_batch(lib, rlca, [batch_record(rlca, call, bufs, storage)], h)
    nsets = len(sets)
    ncalls = len(calls)
    step_bytes = sum(c[3] for c in calls)
    dominant = max(range(ncalls), key=lambda i: calls[i][3])

    stream = torch.cuda.Stream()  # default priority
    # bound launches: step s, call c uses set (s * ncalls + c) % nsets
    cycle = nsets * ncalls // np.gcd(nsets, ncalls)
    steps_per_cycle = cycle // ncalls

    def launches(h):
        """Per step of the rotation cycle, the bound launches: one per call,
        or with --launch batch one rlca_run_batch holding every call."""
        out = []
        for s in range(steps_per_cycle):
            bufs = [sets[(s * ncalls + c) % nsets] for c in range(ncalls)]
            if args.launch == "batch":
                out.append([bind_batch(lib, rlca, [batch_record(rlca, calls[c], bufs[c], storage)
                                                   for c in range(ncalls)], h)])
            else:
                out.append([bind_call(calls[c], bufs[c], h) for c in range(ncalls)])
        return out

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {rlca.STATUS_NAMES.get(st, st)}")

    timed_steps = args.steps
    warm = args.warmup
    with torch.cuda.stream(stream):
        h = stream.cuda_stream
        plan = launches(h)
        if args.launch == "graph":
            # One graph per step of the rotation cycle, captured once, replayed.
            graphs = []
            for s in range(steps_per_cycle):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for fn, a in plan[s]:
                        check(fn(*a), fn.__name__)
                graphs.append(g)
            run_step = lambda s: graphs[s % steps_per_cycle].replay()  # noqa: E731
        else:
            def run_step(s):
                for fn, a in plan[s % steps_per_cycle]:
                    check(fn(*a), fn.__name__)

        for s in range(warm):
            run_step(s)
        torch.cuda.synchronize()

        # whole-step time.  The timed loop does as little host work per step
        # as it can (launches bound beforehand in one flat list, statuses
        # checked after the loop), so that on a slow host the step time
        # measures the library's launches rather than this loop.
        if args.launch == "graph":
            order = [(graphs[(warm + s) % steps_per_cycle].replay, ())
                     for s in range(timed_steps)]
        else:
            order = [fa for s in range(timed_steps) for fa in plan[(warm + s) % steps_per_cycle]]
        statuses = []
        record = statuses.append
        t0 = time.perf_counter()
        e_start = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        e_start.record(stream)
        for fn, a in order:
            record(fn(*a))
        e_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = e_start.elapsed_time(e_end) / timed_steps
        if args.launch != "graph":
            for (fn, _), st in zip(order, statuses):
                check(st, fn.__name__)

        # per-kernel device time: each call variant (and with --launch batch
        # the grouped launch of the whole step) launched back to back `reps`
        # times (rotating sets) between two events on the same stream; the
        # average is elapsed / reps
        reps = max(50, min(timed_steps, 2000))

        def back_to_back(bound):
            for i in range(5):
                fn, a = bound[i % len(bound)]
                check(fn(*a), fn.__name__)
            order = [bound[i % len(bound)] for i in range(reps)]
            statuses = []
            record = statuses.append
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for fn, a in order:
                record(fn(*a))
            e1.record(stream)
            torch.cuda.synchronize()
            for (fn, _), st in zip(order, statuses):
                check(st, fn.__name__)
            return e0.elapsed_time(e1) / reps

        per_call_ms = [back_to_back([bind_call(calls[c], sets[i], h) for i in range(nsets)])
                       for c in range(ncalls)]
        batch_ms = back_to_back([p[0] for p in plan]) if args.launch == "batch" else None

        # the streaming floor of the step (bench_floor.hip), the same rotation
        floor_ms = None
        if os.path.exists(FLOOR_LIB) and host.T % 4 == 0:
            flib = ctypes.CDLL(FLOOR_LIB)
            flib.bench_floor_launch.argtypes = [ctypes.POINTER(_FloorLaunch), ctypes.c_void_p]
            flib.bench_floor_launch.restype = ctypes.c_int
            flib.bench_floor_launch_bytes.restype = ctypes.c_size_t
            if flib.bench_floor_launch_bytes() != ctypes.sizeof(_FloorLaunch):
                raise RuntimeError("bench_floor.so does not match this bench.py")
            recs = [floor_record(calls, [sets[(s * ncalls + c) % nsets] for c in range(ncalls)],
                                 host.num_envs, host.T) for s in range(steps_per_cycle)]
            floor_ms = back_to_back([(flib.bench_floor_launch, (ctypes.byref(r), h))
                                     for r in recs])

        # the pages' protocol: 20 untimed calls, then 5 trials of 50 calls,
        # each call between its own pair of events and followed by a
        # synchronize (full-call time: host launch included); the median of
        # each trial, the minimum over trials
        def pages_protocol(bound):
            for i in range(20):
                fn, a = bound[i % len(bound)]
                check(fn(*a), fn.__name__)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            medians = []
            for trial in range(5):
                times = []
                for i in range(50):
                    fn, a = bound[(trial * 50 + i) % len(bound)]
                    e0.record(stream)
                    check(fn(*a), fn.__name__)
                    e1.record(stream)
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1))
                medians.append(float(np.median(times)))
            return min(medians)

        protocol_ms = {calls[c][0]: pages_protocol([bind_call(calls[c], sets[i], h)
                                                    for i in range(nsets)])
                       for c in range(ncalls)}
        if args.launch == "batch":
            protocol_ms["batch"] = pages_protocol([p[0] for p in plan])

        # same-bytes copy ceiling (cold, rotating): a plain device copy of
        # step_bytes / 2 read + step_bytes / 2 written
        nfl = max(1, step_bytes // 8)
        src = [torch.empty(nfl * 1, dtype=torch.float32, device=device).fill_(1.0)
               for _ in range(max(2, COLD_BYTES // (nfl * 4) + 1))]
        dst = [torch.empty_like(x) for x in src]
        for i in range(10):
            dst[i % len(dst)].copy_(src[i % len(src)])
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        ncopy = 200
        for i in range(ncopy):
            dst[i % len(dst)].copy_(src[i % len(src)])
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1) / ncopy
        copy_gbs = (nfl * 8) / (copy_ms * 1e-3) / 1e9

    nt = host.num_envs * host.T
    return dict(step_ms=step_ms, wall_s=wall, step_bytes=step_bytes, calls=calls,
                per_call_ms=per_call_ms, batch_ms=batch_ms, protocol_ms=protocol_ms,
                floor_ms=floor_ms,
                dominant=dominant, nt=nt,
                nsets=nsets,
                copy_gbs=copy_gbs, copy_bytes=nfl * 8)


# ------------------------------------------------------------------ CPU oracle


def oracle_calls(name, cfg, d):
    """The workload's per-step calls on the fp64 oracle, over rollout d."""
    import oracle

    g = cfg["gamma"]
    lam = cfg.get("lam", 0.95)
    if name in ("gae_td_4096x128", "gae_8x16"):
        fns = [
            lambda: oracle.gae(d.rewards, d.values, d.terminated, None, None, d.bootstrap, g, lam),
            lambda: oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                               d.bootstrap, g, lam),
            lambda: oracle.td_lambda(d.rewards, d.values, d.terminated, None, None, d.bootstrap,
                                     g, lam),
            lambda: oracle.td_lambda(d.rewards, d.values, d.terminated, d.truncated,
                                     d.trunc_values, d.bootstrap, g, lam),
        ]
        return fns[1:2] if name == "gae_8x16" else fns
    if name == "vtrace_4096x256":
        return [lambda: oracle.vtrace(d.rewards, d.values, d.behaviour_logp, d.target_logp,
                                      d.terminated, None, None, d.bootstrap, g, lam,
                                      cfg["rho_bar"], cfg["c_bar"])]
    if name == "retrace_2048x1024":
        return [lambda: oracle.retrace(d.rewards, d.q_values, d.expected_q, d.behaviour_logp,
                                       d.target_logp, d.terminated, d.truncated, d.trunc_values,
                                       d.bootstrap, g, lam, cfg["c_bar"])]
    if name.startswith("long_"):
        return [
            lambda: oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                               d.bootstrap, g, lam),
            lambda: oracle.eligibility_traces(d.rewards, d.terminated, 1, g, lam),
        ]
    if name == "ppo_4096x128":
        def ppo_step():
            adv, _ = oracle.gae(d.rewards, d.values, d.terminated, d.truncated, d.trunc_values,
                                d.bootstrap, g, lam)
            stats = oracle.mean_std(adv)
            oracle.ppo_clip_loss(adv.astype(np.float32), d.target_logp, d.behaviour_logp, stats,
                                 cfg["clip_eps"], 1e-8)
        return [ppo_step]
    return [
        lambda: oracle.discounted_returns(d.rewards, d.dones, None, None, d.bootstrap, g),
        lambda: oracle.eligibility_traces(d.increments, d.starts, 0, g, lam),
        lambda: oracle.episodic_prefix_sum(d.rewards, d.starts, 0),
        lambda: oracle.episodic_prefix_sum(d.ints, d.starts, 0),
    ]


def _rows(d, lo, hi):
    """Rows lo..hi of a rollout (every per-env array sliced, views only)."""
    import dataclasses

    out = {}
    for f in dataclasses.fields(d):
        v = getattr(d, f.name)
        if isinstance(v, np.ndarray) and v.shape[:1] == (d.num_envs,):
            v = v[lo:hi]
        out[f.name] = v
    out["num_envs"] = hi - lo
    return dataclasses.replace(d, **out)


def _oracle_passes(name, lo, hi, seconds):
    """Worker: rows lo..hi of the named workload through the oracle, repeated
    for about `seconds`; returns (passes, seconds taken)."""
    sys.path.insert(0, ROOT)
    from linear_recurrence_scan_row_amd import workloads

    cfg = dict(workloads.CONFIGS[name])
    d = _rows(workloads.make(name), lo, hi)
    fns = oracle_calls(name, cfg, d)
    for f in fns:   # warm-up (also builds the library if needed)
        f()
    passes = 0
    t0 = time.perf_counter()
    while True:
        for f in fns:
            f()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return passes, el


def run_cpu_baseline(name, cfg, host, seconds, workers=1, step_bytes=None):
    """The fp64 sequential oracle on this host's CPU over the same rollout and
    calls, repeated for about `seconds`.  workers > 1 splits the rows evenly
    over that many worker processes (fresh interpreters, no GPU state) that
    run at the same time.  With `step_bytes` (the GPU step's algorithmic
    bytes) the result also carries the same byte model's GB/s, for context."""
    d = host
    nfns = len(oracle_calls(name, cfg, d))
    nt = d.num_envs * d.T

    def with_gbs(rec):
        if step_bytes is not None:   # passes per second times the bytes of one pass
            rec["gbs"] = round(rec["value"] / (nfns * nt) * step_bytes / 1e9, 3)
        return rec

    if workers == 1:
        passes, el = _oracle_passes(name, 0, d.num_envs, seconds)
        return with_gbs(dict(value=passes * nfns * nt / el, unit="env-steps/s", cores=1,
                             kind="oracle",
                             sample=(f"full {d.num_envs}x{d.T} rollout, {nfns} estimator calls "
                                     f"per pass, {passes} passes in {el:.1f} s, one thread, "
                                     f"fp64 sequential C")))
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    bounds = np.linspace(0, d.num_envs, workers + 1).astype(int)
    jobs = [(bounds[k], bounds[k + 1]) for k in range(workers) if bounds[k + 1] > bounds[k]]
    with ProcessPoolExecutor(len(jobs), mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_passes, [name] * len(jobs), [lo for lo, _ in jobs],
                          [hi for _, hi in jobs], [seconds] * len(jobs)))
    steps = sum(p * nfns * (hi - lo) * d.T for (p, _), (lo, hi) in zip(res, jobs))
    el = max(e for _, e in res)
    return with_gbs(dict(value=float(steps / el), unit="env-steps/s", cores=len(jobs),
                         kind="oracle",
                         sample=(f"full {d.num_envs}x{d.T} rollout, {nfns} estimator calls per "
                                 f"pass, rows split over {len(jobs)} worker processes running "
                                 f"together for {el:.1f} s, fp64 sequential C")))


# ------------------------------------------------------------------ traffic


def profiled_times(workload, dtype):
    """(step_avg_us, {call: avg_us}, summary file) from the committed rocprofv3
    kernel-trace summary of this workload, or (None, {}, file) when it is
    missing or the kernel source changed since it was taken."""
    name = f"kernels_{workload}" + ("" if dtype == "f32" else f"_{dtype}") + ".md"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None, {}, name
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from profiling import source_digest

    if kv.get("source_digest") != source_digest():
        return None, {}, name
    calls = {k[len("call_avg_us."):]: float(v) for k, v in kv.items()
             if k.startswith("call_avg_us.")}
    step = float(kv["step_avg_us"]) if "step_avg_us" in kv else None
    return step, calls, name


def measured_traffic(kernel_name, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the summary is missing or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from profiling import source_digest

    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ size sweep

SWEEP_WARMUP_S = 0.2   # untimed launches before each point's trials

# (num_envs, T, estimators) of each sweep grid: "sizes" spans the rollout
# shapes of the workloads above; "long" spans few long rows on both sides of
# the chunked path's bounds (backward rows of 16384 steps or more, fewer than
# 128; forward rows of 32768 steps or more, fewer than 160, and fewer than
# 208 from 65536 steps on: 127, 159 and 207 rows are chunked, 128, 160 and
# 208 take one workgroup per row).
SWEEP_GRIDS = {
    "sizes": ((1024, 4096, 16384, 65536), (128, 512, 2048),
              ("gae+trunc", "retrace+trunc", "eligibility")),
    "long": ((1, 8, 16, 32, 64, 96, 127, 128, 159, 160, 192, 207, 208, 256, 384),
             (4100, 8192, 12288, 16384, 32768, 65536, 131072, 524288),
             ("gae+trunc", "eligibility")),
}


def run_sweep(args):
    """Effective GB/s of GAE with truncation (22 B/step), Retrace with
    truncation (30 B/step) and eligibility traces (9 B/step) over the grid of
    shapes `args.sweep` names; one JSON line per point.  Rollouts are drawn on
    the device with a seeded torch generator (values: N(0,1) and U(0,1);
    flags: Bernoulli 0.01 and 0.005); only throughput is measured here."""
    import torch
    from linear_recurrence_scan_row_amd import rlca

    lib = rlca.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    gen = torch.Generator(device=dev)
    envs, steps, estimators = SWEEP_GRIDS[args.sweep]
    for n in envs:
        for t in steps:
            nt = n * t
            shape = (n, t)
            specs = [
                ("gae+trunc", 22, ("r", "v", "term", "trunc", "tv", "b"), ("o0", "o1")),
                ("retrace+trunc", 30,
                 ("r", "v", "eq", "mu", "pi", "term", "trunc", "tv", "b"), ("o0",)),
                ("eligibility", 9, ("x", "start"), ("o0",)),
            ]
            for name, bps, ins, outs in [x for x in specs if x[0] in estimators]:
                call_bytes = nt * bps + (4 * n if "b" in ins else 0)
                per_set = nt * (4 * sum(1 for k in ins if k not in ("term", "trunc", "start"))
                                + sum(1 for k in ins if k in ("term", "trunc", "start"))
                                + 4 * len(outs))
                nsets = int(min(max(2, -(-COLD_BYTES // call_bytes) + 1),
                                max(2, (48 << 30) // per_set)))
                gen.manual_seed(n * 131 + t)
                sets = []
                for _ in range(nsets):
                    s = {}
                    for k in ins:
                        if k in ("term", "trunc", "start"):
                            p = 0.005 if k == "trunc" else 0.01
                            s[k] = (torch.rand(shape, generator=gen, device=dev) < p).to(torch.uint8)
                        elif k == "b":
                            s[k] = torch.randn(n, generator=gen, device=dev)
                        elif k == "x":
                            s[k] = torch.rand(shape, generator=gen, device=dev)
                        else:
                            s[k] = torch.randn(shape, generator=gen, device=dev)
                    for k in outs:
                        s[k] = torch.empty(shape, device=dev)
                    sets.append(s)
                torch.cuda.synchronize()
                h = stream.cuda_stream

                def bound(s):
                    """(entry point, arguments) of one launch on set s, bound
                    before timing so the timed loop makes one ctypes call."""
                    if name == "gae+trunc":
                        return lib.rlca_gae, (s["r"].data_ptr(), s["v"].data_ptr(),
                                              s["term"].data_ptr(), s["trunc"].data_ptr(),
                                              s["tv"].data_ptr(), s["b"].data_ptr(), 0.99, 0.95,
                                              n, t, s["o0"].data_ptr(), s["o1"].data_ptr(), h)
                    if name == "retrace+trunc":
                        return lib.rlca_retrace, (*[s[k].data_ptr() for k in ins], 0.99, 0.95,
                                                  1.0, n, t, s["o0"].data_ptr(), h)
                    return lib.rlca_eligibility_traces, (s["x"].data_ptr(), s["start"].data_ptr(),
                                                         0, 0.99, 0.9, n, t, s["o0"].data_ptr(),
                                                         h)

                plan = [bound(s) for s in sets]
                batch = max(20, min(400, int(2e9 // call_bytes)))
                trials = []
                with torch.cuda.stream(stream):
                    # warm up for at least SWEEP_WARMUP_S of launches (a
                    # quarter of a trial alone was too short for the clocks
                    # to rise at the small points: 4096 x 128 GAE + trunc
                    # read 4.8 us there against 3.8 us after the bench's
                    # warm-up), then three trials of `batch` back-to-back
                    # launches; the fastest trial is reported (the pages'
                    # protocol also keeps a minimum), so that a transient
                    # stall of the host or the GPU during one trial does not
                    # stand for the kernel
                    warm_until = time.perf_counter() + SWEEP_WARMUP_S
                    while True:
                        for i in range(max(20, batch // 4)):
                            fn, a = plan[i % nsets]
                            if fn(*a) != 0:
                                raise RuntimeError(f"{name} {n}x{t}: launch failed")
                        torch.cuda.synchronize()
                        if time.perf_counter() >= warm_until:
                            break
                    for _ in range(3):
                        order = [plan[i % nsets] for i in range(batch)]
                        statuses = []
                        record = statuses.append
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for fn, a in order:
                            record(fn(*a))
                        e1.record(stream)
                        torch.cuda.synchronize()
                        if any(statuses):
                            raise RuntimeError(f"{name} {n}x{t}: launch failed")
                        trials.append(e0.elapsed_time(e1) / batch * 1e3)
                us = min(trials)
                gbs = call_bytes / (us * 1e-6) / 1e9
                print(json.dumps({"sweep": name, "num_envs": n, "T": t, "us": round(us, 3),
                                  "bytes": call_bytes, "gbs": round(gbs, 1),
                                  "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                                  "env_steps_per_s": nt / (us * 1e-6), "sets": nsets,
                                  "trials_us": [round(x, 3) for x in trials]}),
                      flush=True)
                del sets
                torch.cuda.empty_cache()


# ------------------------------------------------------------------ main


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first: enough to bring the GPU clocks up (with 20 "
                         "the timed steps ran 1.2%% slower at 4096x128)")
    ap.add_argument("--workload", default="gae_td_4096x128")
    ap.add_argument("--launch", choices=("batch", "graph", "eager"), default="batch")
    ap.add_argument("--dtype", choices=tuple(STORAGE), default="f32",
                    help="storage type of the real-valued arrays (arithmetic is fp32)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", nargs="?", const="sizes", choices=tuple(SWEEP_GRIDS),
                    help="print one JSON line per (num_envs, T, estimator) of a size sweep "
                         "(grid 'sizes' by default, or 'long': few long rows)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library's hot path has no multi-GPU "
              f"step (rows are independent; sharding over envs needs no communication). "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    sys.path.insert(0, ROOT)
    if args.sweep:
        run_sweep(args)
        return
    from linear_recurrence_scan_row_amd import workloads

    cfg = dict(workloads.CONFIGS[args.workload])
    host = workloads.make(args.workload)
    res = run_gpu(args, args.workload, cfg, host)

    step_s = res["step_ms"] * 1e-3
    ncalls = len(res["calls"])
    value = res["step_bytes"] / step_s / 1e9
    if res["batch_ms"] is not None and ncalls > 1:
        # one grouped launch runs the whole step: it is the dominant kernel
        # (a one-call batch runs the call's own kernel, timed per call)
        dom_name, dom_bytes, dom_ms = "batch", res["step_bytes"], res["batch_ms"]
    else:
        dcall = res["calls"][res["dominant"]]
        dom_name, dom_bytes, dom_ms = dcall[0], dcall[3], res["per_call_ms"][res["dominant"]]
    achieved_event = dom_bytes / (dom_ms * 1e-3) / 1e9
    tag = dom_name.replace("+", "_") + ("" if args.dtype == "f32" else "_" + args.dtype)
    traffic = measured_traffic(tag, args.workload)
    # the dominant kernel's average duration from the committed rocprofv3
    # kernel trace of this workload (a step of one grouped launch, or the
    # one call), when that summary was taken on the current kernel sources;
    # the tracer runs dispatches one at a time, so it reads a little above
    # the back-to-back event time, which is kept beside it
    prof_step_us, prof_calls, prof_file = profiled_times(args.workload, args.dtype)
    prof_us = prof_step_us if dom_name == "batch" else prof_calls.get(dom_name)
    if prof_us is not None:
        achieved, avg_us, source = dom_bytes / (prof_us * 1e-6) / 1e9, prof_us, \
            f"rocprofv3 kernel trace, profiles/{prof_file}"
    else:
        achieved, avg_us, source = achieved_event, dom_ms * 1e3, "HIP events, back to back"

    calls_out = {}
    for i, c in enumerate(res["calls"]):
        ms = res["per_call_ms"][i]
        calls_out[c[0]] = dict(us=round(ms * 1e3, 3), bytes=c[3],
                               gbs=round(c[3] / (ms * 1e-3) / 1e9, 1),
                               env_steps_per_s=res["nt"] / (ms * 1e-3))

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["step_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded numpy rollouts; cold-cache rotation over "
                f"{res['nsets']} HBM-resident copies)",
        "config": {
            "workload": args.workload,
            "num_envs": host.num_envs,
            "T": host.T,
            "calls_per_step": [c[0] for c in res["calls"]],
            "launch": args.launch,
            "storage": args.dtype,
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        # independent estimator calls each cover the rollout; the fused PPO
        # calls form one pipeline over it
        "env_steps_per_s": (1 if args.workload == "ppo_4096x128" else ncalls) * res["nt"] / step_s,
        "bytes_per_step": res["step_bytes"],
        "calls": calls_out,
        "full_call_us": {k: round(v * 1e3, 3) for k, v in res["protocol_ms"].items()},
        "copy_ceiling": {"gbs": round(res["copy_gbs"], 1), "bytes": res["copy_bytes"],
                         "kind": "torch device copy, cold rotation, same bytes moved",
                         "value_over_copy": round(value / res["copy_gbs"], 4)},
        "roofline": {
            "kernel": dom_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": dom_bytes,
            "avg_us": round(avg_us, 3),
            "source": source,
            "achieved_event": round(achieved_event, 1),
            "frac_event": round(achieved_event / HBM_PEAK_GBS, 4),
            "avg_us_event": round(dom_ms * 1e3, 3),
        },
    }
    if res["floor_ms"] is not None:
        out["floor"] = {
            "us": round(res["floor_ms"] * 1e3, 3),
            "gbs": round(res["step_bytes"] / (res["floor_ms"] * 1e-3) / 1e9, 1),
            "kind": "bench_floor.hip: the step's bytes, the library's tiling and access widths, "
                    "no arithmetic, one launch per step, same cold rotation",
            "value_over_floor": round(res["floor_ms"] / res["step_ms"], 4),
        }
    # the metric names the GAE call: its own kernel's roofline, beside the step's
    names = [c[0] for c in res["calls"]]
    if "gae" in names and ncalls > 1:
        i = names.index("gae")
        ms, b = res["per_call_ms"][i], res["calls"][i][3]
        g_prof = prof_calls.get("gae")
        g_us = g_prof if g_prof is not None else ms * 1e3
        out["roofline_gae_call"] = {
            "kernel": "gae (one call, its own launch)",
            "achieved": round(b / (g_us * 1e-6) / 1e9, 1),
            "frac": round(b / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "avg_us": round(g_us, 3),
            "source": (f"rocprofv3 kernel trace, profiles/{prof_file}" if g_prof is not None
                       else "HIP events, back to back"),
            "avg_us_event": round(ms * 1e3, 3),
            "traffic": measured_traffic("gae" + ("" if args.dtype == "f32" else "_" + args.dtype),
                                        args.workload),
            "algorithmic_bytes": b,
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(args.workload, cfg, host, args.cpu_seconds,
                                               step_bytes=res["step_bytes"])
        try:
            nproc = int(subprocess.run(["nproc"], capture_output=True, text=True).stdout)
        except (OSError, ValueError):
            nproc = None
        out["host_cores"] = {"affinity": len(os.sched_getaffinity(0)), "nproc": nproc,
                             "cpu_count": os.cpu_count()}
        # the same oracle with the rows split over the host's cores (at most
        # 16, the CPU share of one GPU), for context
        cores = min(16, len(os.sched_getaffinity(0)))
        if cores > 1:
            out["cpu_baseline_all_cores"] = run_cpu_baseline(args.workload, cfg, host,
                                                             args.cpu_seconds / 2, cores,
                                                             step_bytes=res["step_bytes"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
