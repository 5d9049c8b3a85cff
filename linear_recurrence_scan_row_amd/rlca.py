"""Thin ctypes binding of librlca.so (the C ABI declared in include/rlca.h).

Argument marshalling only: shape / dtype / device checks, output allocation
through torch, and the current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no CPU fallback, and a missing library
raises instead of degrading.
"""
from __future__ import annotations

import ctypes
import threading
import inspect
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librlca.so")

RLCA_OK = 0
STATUS_NAMES = {
    0: "RLCA_OK", 1: "RLCA_ERR_NULL_POINTER", 2: "RLCA_ERR_INVALID_SIZE",
    3: "RLCA_ERR_INVALID_VALUE", 4: "RLCA_ERR_ALIASING", 5: "RLCA_ERR_MISALIGNED",
    6: "RLCA_ERR_HIP",
}
RESET_ON_START = 0
RESET_AFTER_DONE = 1
RLCA_F32 = 0
RLCA_I32 = 1
RLCA_BF16 = 2
RLCA_F16 = 3
# storage types of real-valued arrays (arithmetic is fp32 for all of them)
REAL_DTYPES = {torch.float32: RLCA_F32, torch.bfloat16: RLCA_BF16, torch.float16: RLCA_F16}
BACKWARD = 0
FORWARD = 1

_p = ctypes.c_void_p
_f = ctypes.c_float
_i64 = ctypes.c_int64
_i = ctypes.c_int
_sz = ctypes.c_size_t


class RlcaCall(ctypes.Structure):
    """One call of a batch (rlca_call in include/rlca.h)."""

    _fields_ = [
        ("op", ctypes.c_int), ("num_envs", ctypes.c_int64), ("T", ctypes.c_int64),
        ("rewards", _p), ("values", _p), ("expected_q", _p), ("behaviour_logp", _p),
        ("target_logp", _p), ("terminated", _p), ("truncated", _p), ("trunc_values", _p),
        ("bootstrap", _p), ("gamma", _f), ("lambda_", _f), ("rho_bar", _f), ("c_bar", _f),
        ("convention", ctypes.c_int), ("dtype", ctypes.c_int), ("direction", ctypes.c_int),
        ("out0", _p), ("out1", _p),
    ]


OP_GAE, OP_TD_LAMBDA, OP_DISCOUNTED, OP_VTRACE, OP_RETRACE, OP_TRACES, OP_PREFIX_SUM, \
    OP_AFFINE = range(8)
MAX_BATCH = 64

# name -> argument types, in the order of include/rlca.h
SIGNATURES = {
    "rlca_gae": [_p, _p, _p, _p, _p, _p, _f, _f, _i64, _i64, _p, _p, _p],
    "rlca_td_lambda": [_p, _p, _p, _p, _p, _p, _f, _f, _i64, _i64, _p, _p],
    "rlca_discounted_returns": [_p, _p, _p, _p, _p, _f, _i64, _i64, _p, _p],
    "rlca_vtrace": [_p, _p, _p, _p, _p, _p, _p, _p, _f, _f, _f, _f, _i64, _i64, _p, _p, _p],
    "rlca_retrace": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _f, _f, _f, _i64, _i64, _p, _p],
    "rlca_eligibility_traces": [_p, _p, _i, _f, _f, _i64, _i64, _p, _p],
    "rlca_episodic_prefix_sum": [_p, _i, _p, _i, _i64, _i64, _p, _p],
    "rlca_affine_scan": [_p, _p, _p, _i, _i64, _i64, _p, _p],
    "rlca_run_batch": [ctypes.POINTER(RlcaCall), _i, _p],
    "rlca_gae_stats": [_p, _p, _p, _p, _p, _p, _f, _f, _i64, _i64, _p, _p, _p, _p, _sz, _p],
    "rlca_ppo_clip_loss": [_p, _p, _p, _p, _f, _f, _i64, _i64, _p, _p, _p, _sz, _p],
    "rlca_gae_stats_noalloc": [_p, _p, _p, _p, _p, _p, _f, _f, _i64, _i64, _p, _p, _p, _p],
}
# workspace-size queries (return size_t)
SIZE_QUERIES = {
    "rlca_gae_stats_workspace_size": [_i64, _i64],
    "rlca_ppo_clip_loss_workspace_size": [_i64, _i64],
}

_lib = None


class RlcaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} "
                         f"({lib().rlca_status_string(status).decode()})")


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_recurrence_scan_row_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in SIZE_QUERIES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = _sz
        l.rlca_status_string.argtypes = [ctypes.c_int]
        l.rlca_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


# The current stream's raw handle: torch's own getter is about 25x cheaper
# than building a torch.cuda.Stream per call; the public API is the fallback.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(dev: torch.device) -> int:
    if _raw_current_stream is not None:
        return _raw_current_stream(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, fn: str):
    if status != RLCA_OK:
        raise RlcaError(status, fn)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_FLAG_DTYPES = (torch.uint8, torch.bool)


def _steps(name, t, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    # every check in one expression first; the detailed ones below name the
    # failure
    if (t.device == device and t.shape == shape and t.is_contiguous()
            and (t.dtype in _FLAG_DTYPES if dtype == "flag" else t.dtype == dtype)):
        return t
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype == "flag":
        if t.dtype not in (torch.uint8, torch.bool):
            raise TypeError(f"{name} must be uint8 or bool, got {t.dtype}")
    elif t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _rollout_shape(rewards: torch.Tensor):
    if rewards.dim() != 2:
        raise ValueError("per-step inputs are [num_envs, T]")
    if rewards.device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    return tuple(rewards.shape), rewards.device


def _real_dtype(name, t: torch.Tensor):
    """The storage type of a call's real-valued arrays, taken from its first
    real input: float32, bfloat16 or float16."""
    if t.dtype not in REAL_DTYPES:
        raise TypeError(f"{name} must be float32, bfloat16 or float16, got {t.dtype}")
    return t.dtype


def _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev, fdt):
    term = _steps("terminated", terminated, shape, "flag", dev)
    trunc = _steps("truncated", truncated, shape, "flag", dev, optional=True)
    tv = _steps("trunc_values", trunc_values, shape, fdt, dev, optional=True)
    if trunc is not None and tv is None:
        raise ValueError("trunc_values is required when truncated is given")
    boot = _steps("bootstrap", bootstrap, shape[:1], fdt, dev, optional=True)
    return term, trunc, tv if trunc is not None else None, boot


def _out(out, shape, dev, dtype=torch.float32, name="out"):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _steps(name, out, shape, dtype, dev)


class _Prepared:
    """One checked call: its op, shape and device, the rlca_call fields it sets
    (tensors for pointers), and the output tensor(s) handed back to the caller."""

    __slots__ = ("op", "shape", "dev", "fields", "result")

    def __init__(self, op, shape, dev, result, **fields):
        self.op, self.shape, self.dev, self.result, self.fields = op, shape, dev, result, fields

    @property
    def f32(self):
        return self.fields.get("dtype", RLCA_F32) == RLCA_F32

    def arg(self, name, default=None):
        v = self.fields.get(name, default)
        return _ptr(v) if isinstance(v, torch.Tensor) else v

    def stream(self):
        return _current_stream(self.dev)


def _prepare_gae(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
                 gamma=0.99, lam=0.95, with_returns=True, advantages=None, returns=None):
    shape, dev = _rollout_shape(rewards)
    fdt = _real_dtype("rewards", rewards)
    r = _steps("rewards", rewards, shape, fdt, dev)
    v = _steps("values", values, shape, fdt, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev,
                                      fdt)
    adv = _out(advantages, shape, dev, fdt, name="advantages")
    ret = _out(returns, shape, dev, fdt, name="returns") if with_returns else None
    return _Prepared(OP_GAE, shape, dev, (adv, ret), rewards=r, values=v, terminated=term,
                     truncated=trunc, trunc_values=tv, bootstrap=boot, gamma=gamma, lambda_=lam,
                     out0=adv, out1=ret, dtype=REAL_DTYPES[fdt])


def _prepare_td_lambda(rewards, values, terminated, truncated=None, trunc_values=None,
                       bootstrap=None, gamma=0.99, lam=0.95, out=None):
    shape, dev = _rollout_shape(rewards)
    fdt = _real_dtype("rewards", rewards)
    r = _steps("rewards", rewards, shape, fdt, dev)
    v = _steps("values", values, shape, fdt, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev,
                                      fdt)
    g = _out(out, shape, dev, fdt)
    return _Prepared(OP_TD_LAMBDA, shape, dev, g, rewards=r, values=v, terminated=term,
                     truncated=trunc, trunc_values=tv, bootstrap=boot, gamma=gamma, lambda_=lam,
                     out0=g, dtype=REAL_DTYPES[fdt])


def _prepare_discounted_returns(rewards, terminated, truncated=None, trunc_values=None,
                                bootstrap=None, gamma=0.99, out=None):
    shape, dev = _rollout_shape(rewards)
    fdt = _real_dtype("rewards", rewards)
    r = _steps("rewards", rewards, shape, fdt, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev,
                                      fdt)
    g = _out(out, shape, dev, fdt)
    return _Prepared(OP_DISCOUNTED, shape, dev, g, rewards=r, terminated=term, truncated=trunc,
                     trunc_values=tv, bootstrap=boot, gamma=gamma, out0=g,
                     dtype=REAL_DTYPES[fdt])


def _prepare_vtrace(rewards, values, behaviour_logp, target_logp, terminated, truncated=None,
                    trunc_values=None, bootstrap=None, gamma=0.99, lam=1.0, rho_bar=1.0,
                    c_bar=1.0, with_pg=True, vs=None, pg_advantages=None):
    shape, dev = _rollout_shape(rewards)
    fdt = _real_dtype("rewards", rewards)
    r = _steps("rewards", rewards, shape, fdt, dev)
    v = _steps("values", values, shape, fdt, dev)
    mu = _steps("behaviour_logp", behaviour_logp, shape, fdt, dev)
    pi = _steps("target_logp", target_logp, shape, fdt, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev,
                                      fdt)
    o_vs = _out(vs, shape, dev, fdt, name="vs")
    o_pg = _out(pg_advantages, shape, dev, fdt, name="pg_advantages") if with_pg else None
    return _Prepared(OP_VTRACE, shape, dev, (o_vs, o_pg), rewards=r, values=v,
                     behaviour_logp=mu, target_logp=pi, terminated=term, truncated=trunc,
                     trunc_values=tv, bootstrap=boot, gamma=gamma, lambda_=lam, rho_bar=rho_bar,
                     c_bar=c_bar, out0=o_vs, out1=o_pg, dtype=REAL_DTYPES[fdt])


def _prepare_retrace(rewards, q_values, expected_q, behaviour_logp, target_logp, terminated,
                     truncated=None, trunc_values=None, bootstrap=None, gamma=0.99, lam=0.95,
                     c_bar=1.0, out=None):
    shape, dev = _rollout_shape(rewards)
    fdt = _real_dtype("rewards", rewards)
    r = _steps("rewards", rewards, shape, fdt, dev)
    q = _steps("q_values", q_values, shape, fdt, dev)
    eq = _steps("expected_q", expected_q, shape, fdt, dev)
    mu = _steps("behaviour_logp", behaviour_logp, shape, fdt, dev)
    pi = _steps("target_logp", target_logp, shape, fdt, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev,
                                      fdt)
    o = _out(out, shape, dev, fdt)
    return _Prepared(OP_RETRACE, shape, dev, o, rewards=r, values=q, expected_q=eq,
                     behaviour_logp=mu, target_logp=pi, terminated=term, truncated=trunc,
                     trunc_values=tv, bootstrap=boot, gamma=gamma, lambda_=lam, c_bar=c_bar,
                     out0=o, dtype=REAL_DTYPES[fdt])


def _prepare_eligibility_traces(increments, flags, convention=RESET_ON_START, gamma=0.99,
                                lam=0.9, out=None):
    shape, dev = _rollout_shape(increments)
    fdt = _real_dtype("increments", increments)
    x = _steps("increments", increments, shape, fdt, dev)
    f = _steps("flags", flags, shape, "flag", dev)
    o = _out(out, shape, dev, fdt)
    return _Prepared(OP_TRACES, shape, dev, o, rewards=x, terminated=f,
                     convention=int(convention), gamma=gamma, lambda_=lam, out0=o,
                     dtype=REAL_DTYPES[fdt])


def _prepare_episodic_prefix_sum(x, flags, convention=RESET_ON_START, out=None):
    shape, dev = _rollout_shape(x)
    if x.dtype == torch.int32:
        dtype = RLCA_I32
    elif x.dtype in REAL_DTYPES:
        dtype = REAL_DTYPES[x.dtype]
    else:
        raise TypeError(f"x must be float32, bfloat16, float16 or int32, got {x.dtype}")
    xs = _steps("x", x, shape, x.dtype, dev)
    f = _steps("flags", flags, shape, "flag", dev)
    o = _out(out, shape, dev, dtype=x.dtype)
    return _Prepared(OP_PREFIX_SUM, shape, dev, o, rewards=xs, terminated=f,
                     convention=int(convention), dtype=dtype, out0=o)


def _prepare_affine_scan(alpha, beta, carry=None, direction=BACKWARD, out=None):
    shape, dev = _rollout_shape(alpha)
    fdt = _real_dtype("alpha", alpha)
    a = _steps("alpha", alpha, shape, fdt, dev)
    b = _steps("beta", beta, shape, fdt, dev)
    c = _steps("carry", carry, shape[:1], fdt, dev, optional=True)
    o = _out(out, shape, dev, fdt)
    return _Prepared(OP_AFFINE, shape, dev, o, rewards=a, values=b, bootstrap=c,
                     direction=int(direction), out0=o, dtype=REAL_DTYPES[fdt])


# Workspaces of the fused consumers, one per (device, stream), zero-filled
# when allocated: every call leaves its workspace zero-filled again (its
# ticket counter back at zero), so calls on one stream, which run in order,
# share it.  Grown by replacement when a call needs more.
_workspaces = {}
_workspaces_lock = threading.Lock()


def _workspace(query, shape, dev, stream):
    nbytes = getattr(lib(), query)(*shape)
    key = (dev.index, stream)
    with _workspaces_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            # enqueued on the current stream, the one the call runs on
            ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=dev)
            _workspaces[key] = ws
    return ws, ws.numel()


def gae_stats(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
              gamma=0.99, lam=0.95, with_returns=True, advantages=None, returns=None,
              stats=None):
    """GAE (float32) plus the mean and sample std of the advantages over all
    steps, reduced in the same pass.  Returns (advantages, returns|None,
    stats), stats a float64 tensor [mean, std] on the device."""
    p = _prepare_gae(rewards, values, terminated, truncated, trunc_values, bootstrap, gamma,
                     lam, with_returns, advantages, returns)
    if not p.f32:
        raise TypeError("gae_stats takes float32 arrays")
    st = _out(stats, (2,), p.dev, torch.float64, name="stats")
    h = p.stream()
    ws, nbytes = _workspace("rlca_gae_stats_workspace_size", p.shape, p.dev, h)
    _check(lib().rlca_gae_stats(p.arg("rewards"), p.arg("values"), p.arg("terminated"),
                                p.arg("truncated"), p.arg("trunc_values"), p.arg("bootstrap"),
                                p.arg("gamma"), p.arg("lambda_"), *p.shape, p.arg("out0"),
                                p.arg("out1"), _ptr(st), _ptr(ws), nbytes, h),
           "rlca_gae_stats")
    return p.result + (st,)


def gae_stats_noalloc(rewards, values, terminated, truncated=None, trunc_values=None,
                      bootstrap=None, gamma=0.99, lam=0.95, with_returns=True, advantages=None,
                      returns=None, stats=None):
    """gae_stats without a workspace: the partial sums go to the library's own
    static device buffer (rlca_gae_stats_noalloc).  Pass advantages, returns
    and stats tensors to make the call allocate nothing at all."""
    p = _prepare_gae(rewards, values, terminated, truncated, trunc_values, bootstrap, gamma,
                     lam, with_returns, advantages, returns)
    if not p.f32:
        raise TypeError("gae_stats_noalloc takes float32 arrays")
    st = _out(stats, (2,), p.dev, torch.float64, name="stats")
    _check(lib().rlca_gae_stats_noalloc(p.arg("rewards"), p.arg("values"), p.arg("terminated"),
                                        p.arg("truncated"), p.arg("trunc_values"),
                                        p.arg("bootstrap"), p.arg("gamma"), p.arg("lambda_"),
                                        *p.shape, p.arg("out0"), p.arg("out1"), _ptr(st),
                                        p.stream()),
           "rlca_gae_stats_noalloc")
    return p.result + (st,)


def ppo_clip_loss(advantages, logp_new, logp_old, stats=None, clip_eps=0.2, norm_eps=1e-8,
                  with_grad=True, grad=None):
    """PPO clipped-surrogate loss (float64 scalar tensor on the device) and its
    gradient in logp_new (float32, or None).  stats = [mean, std] (float64,
    e.g. from gae_stats) normalizes the advantages on the fly."""
    shape, dev = _rollout_shape(advantages)
    a = _steps("advantages", advantages, shape, torch.float32, dev)
    new = _steps("logp_new", logp_new, shape, torch.float32, dev)
    old = _steps("logp_old", logp_old, shape, torch.float32, dev)
    st = _steps("stats", stats, (2,), torch.float64, dev, optional=True)
    g = _out(grad, shape, dev, name="grad") if with_grad else None
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    h = _current_stream(dev)
    ws, nbytes = _workspace("rlca_ppo_clip_loss_workspace_size", shape, dev, h)
    _check(lib().rlca_ppo_clip_loss(_ptr(a), _ptr(st), _ptr(new), _ptr(old), clip_eps, norm_eps,
                                    *shape, _ptr(g), _ptr(loss), _ptr(ws), nbytes, h),
           "rlca_ppo_clip_loss")
    return loss, g


def _run_alone(p: _Prepared):
    """Enqueue one bf16 / fp16 call: its entry point is rlca_run_batch (the
    single-call entry points are fp32)."""
    b = Batch()
    b._add(p)
    b.run()
    return p.result


def _takes_args_of(prepare):
    """Give a wrapper the signature of the _prepare_* function it forwards to."""
    def deco(fn):
        fn.__signature__ = inspect.signature(prepare)
        return fn
    return deco


@_takes_args_of(_prepare_gae)
def gae(*args, **kwargs):
    """GAE advantages (and value targets adv + V).  Returns (advantages, returns|None)."""
    p = _prepare_gae(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_gae(p.arg("rewards"), p.arg("values"), p.arg("terminated"),
                          p.arg("truncated"), p.arg("trunc_values"), p.arg("bootstrap"),
                          p.arg("gamma"), p.arg("lambda_"), *p.shape, p.arg("out0"),
                          p.arg("out1"), p.stream()), "rlca_gae")
    return p.result


@_takes_args_of(_prepare_td_lambda)
def td_lambda(*args, **kwargs):
    """TD(lambda) returns."""
    p = _prepare_td_lambda(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_td_lambda(p.arg("rewards"), p.arg("values"), p.arg("terminated"),
                                p.arg("truncated"), p.arg("trunc_values"), p.arg("bootstrap"),
                                p.arg("gamma"), p.arg("lambda_"), *p.shape, p.arg("out0"),
                                p.stream()), "rlca_td_lambda")
    return p.result


@_takes_args_of(_prepare_discounted_returns)
def discounted_returns(*args, **kwargs):
    """Discounted returns (Monte-Carlo when bootstrap is None)."""
    p = _prepare_discounted_returns(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_discounted_returns(p.arg("rewards"), p.arg("terminated"),
                                         p.arg("truncated"), p.arg("trunc_values"),
                                         p.arg("bootstrap"), p.arg("gamma"), *p.shape,
                                         p.arg("out0"), p.stream()), "rlca_discounted_returns")
    return p.result


@_takes_args_of(_prepare_vtrace)
def vtrace(*args, **kwargs):
    """V-Trace targets and policy-gradient advantages.  Returns (vs, pg|None)."""
    p = _prepare_vtrace(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_vtrace(p.arg("rewards"), p.arg("values"), p.arg("behaviour_logp"),
                             p.arg("target_logp"), p.arg("terminated"), p.arg("truncated"),
                             p.arg("trunc_values"), p.arg("bootstrap"), p.arg("gamma"),
                             p.arg("lambda_"), p.arg("rho_bar"), p.arg("c_bar"), *p.shape,
                             p.arg("out0"), p.arg("out1"), p.stream()), "rlca_vtrace")
    return p.result


@_takes_args_of(_prepare_retrace)
def retrace(*args, **kwargs):
    """Retrace(lambda) targets Q^ret."""
    p = _prepare_retrace(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_retrace(p.arg("rewards"), p.arg("values"), p.arg("expected_q"),
                              p.arg("behaviour_logp"), p.arg("target_logp"),
                              p.arg("terminated"), p.arg("truncated"), p.arg("trunc_values"),
                              p.arg("bootstrap"), p.arg("gamma"), p.arg("lambda_"),
                              p.arg("c_bar"), *p.shape, p.arg("out0"), p.stream()),
           "rlca_retrace")
    return p.result


@_takes_args_of(_prepare_eligibility_traces)
def eligibility_traces(*args, **kwargs):
    """Accumulating eligibility traces, forward in time."""
    p = _prepare_eligibility_traces(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_eligibility_traces(p.arg("rewards"), p.arg("terminated"),
                                         p.arg("convention"), p.arg("gamma"),
                                         p.arg("lambda_"), *p.shape, p.arg("out0"),
                                         p.stream()), "rlca_eligibility_traces")
    return p.result


@_takes_args_of(_prepare_episodic_prefix_sum)
def episodic_prefix_sum(*args, **kwargs):
    """Inclusive segmented prefix sum over float32 or int32 input (int32 wraps)."""
    p = _prepare_episodic_prefix_sum(*args, **kwargs)
    _check(lib().rlca_episodic_prefix_sum(p.arg("rewards"), p.arg("dtype"), p.arg("terminated"),
                                          p.arg("convention"), *p.shape, p.arg("out0"),
                                          p.stream()), "rlca_episodic_prefix_sum")
    return p.result


@_takes_args_of(_prepare_affine_scan)
def affine_scan(*args, **kwargs):
    """A_t = alpha_t + beta_t * A_{t+1} (BACKWARD, A_T = carry) or
    A_t = alpha_t + beta_t * A_{t-1} (FORWARD, A_{-1} = carry), float32."""
    p = _prepare_affine_scan(*args, **kwargs)
    if not p.f32:
        return _run_alone(p)
    _check(lib().rlca_affine_scan(p.arg("rewards"), p.arg("values"), p.arg("bootstrap"),
                                  p.arg("direction"), *p.shape, p.arg("out0"), p.stream()),
           "rlca_affine_scan")
    return p.result


def _recorder(prepare):
    def record(self, *args, **kwargs):
        return self._add(prepare(*args, **kwargs))
    record.__name__ = prepare.__name__[len("_prepare_"):]
    params = list(inspect.signature(prepare).parameters.values())
    record.__signature__ = inspect.Signature(
        [inspect.Parameter("self", inspect.Parameter.POSITIONAL_OR_KEYWORD)] + params)
    record.__doc__ = (f"Record a {record.__name__} call (arguments as for the function of "
                      "that name); returns its output tensor(s), filled once run() has been "
                      "enqueued.")
    return record


class Batch:
    """Calls recorded here are enqueued together by run() through
    rlca_run_batch: calls on the vector path share grouped launches (up to 14
    calls per launch), the rest run one launch each.  Each recording method
    checks its arguments like the function of the same name.  No call may
    write what another call of the batch reads or writes (rlca_run_batch
    rejects that), so the calls of one batch are independent."""

    def __init__(self):
        self._calls = []
        self._keep = []
        self._device = None

    def _add(self, p: _Prepared):
        if self._device is None:
            self._device = p.dev
        elif p.dev != self._device:
            raise ValueError("all calls of a batch must be on one device")
        if len(self._calls) >= MAX_BATCH:
            raise ValueError(f"a batch holds at most {MAX_BATCH} calls")
        c = RlcaCall(op=p.op, num_envs=p.shape[0], T=p.shape[1])
        for name in p.fields:
            setattr(c, name, p.arg(name))
        self._calls.append(c)
        self._keep.extend(v for v in p.fields.values() if isinstance(v, torch.Tensor))
        return p.result

    def __len__(self):
        return len(self._calls)

    gae = _recorder(_prepare_gae)
    td_lambda = _recorder(_prepare_td_lambda)
    discounted_returns = _recorder(_prepare_discounted_returns)
    vtrace = _recorder(_prepare_vtrace)
    retrace = _recorder(_prepare_retrace)
    eligibility_traces = _recorder(_prepare_eligibility_traces)
    episodic_prefix_sum = _recorder(_prepare_episodic_prefix_sum)
    affine_scan = _recorder(_prepare_affine_scan)

    def run(self):
        """Enqueue every recorded call on the current stream of their device.
        The batch can be run again; its output tensors are rewritten."""
        if not self._calls:
            return
        arr = (RlcaCall * len(self._calls))(*self._calls)
        stream = _current_stream(self._device)
        _check(lib().rlca_run_batch(arr, len(self._calls), stream), "rlca_run_batch")
