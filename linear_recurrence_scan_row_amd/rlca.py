"""Thin ctypes binding of librlca.so (the C ABI declared in include/rlca.h).

Argument marshalling only: shape / dtype / device checks, output allocation
through torch, and the current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no CPU fallback, and a missing library
raises instead of degrading.
"""
from __future__ import annotations

import ctypes
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
BACKWARD = 0
FORWARD = 1

_p = ctypes.c_void_p
_f = ctypes.c_float
_i64 = ctypes.c_int64
_i = ctypes.c_int

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
        l.rlca_status_string.argtypes = [ctypes.c_int]
        l.rlca_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


def _check(status: int, fn: str):
    if status != RLCA_OK:
        raise RlcaError(status, fn)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _steps(name, t, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
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


def _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev):
    term = _steps("terminated", terminated, shape, "flag", dev)
    trunc = _steps("truncated", truncated, shape, "flag", dev, optional=True)
    tv = _steps("trunc_values", trunc_values, shape, torch.float32, dev, optional=True)
    if trunc is not None and tv is None:
        raise ValueError("trunc_values is required when truncated is given")
    boot = _steps("bootstrap", bootstrap, shape[:1], torch.float32, dev, optional=True)
    return term, trunc, tv if trunc is not None else None, boot


def _out(out, shape, dev, dtype=torch.float32, name="out"):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _steps(name, out, shape, dtype, dev)


def gae(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
        gamma=0.99, lam=0.95, with_returns=True, advantages=None, returns=None):
    """GAE advantages (and value targets adv + V).  Returns (advantages, returns|None)."""
    shape, dev = _rollout_shape(rewards)
    r = _steps("rewards", rewards, shape, torch.float32, dev)
    v = _steps("values", values, shape, torch.float32, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev)
    adv = _out(advantages, shape, dev, name="advantages")
    ret = _out(returns, shape, dev, name="returns") if with_returns else None
    _check(lib().rlca_gae(_ptr(r), _ptr(v), _ptr(term), _ptr(trunc), _ptr(tv), _ptr(boot),
                          gamma, lam, shape[0], shape[1], _ptr(adv), _ptr(ret), _stream(r)),
           "rlca_gae")
    return adv, ret


def td_lambda(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
              gamma=0.99, lam=0.95, out=None):
    """TD(lambda) returns."""
    shape, dev = _rollout_shape(rewards)
    r = _steps("rewards", rewards, shape, torch.float32, dev)
    v = _steps("values", values, shape, torch.float32, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev)
    g = _out(out, shape, dev)
    _check(lib().rlca_td_lambda(_ptr(r), _ptr(v), _ptr(term), _ptr(trunc), _ptr(tv), _ptr(boot),
                                gamma, lam, shape[0], shape[1], _ptr(g), _stream(r)),
           "rlca_td_lambda")
    return g


def discounted_returns(rewards, terminated, truncated=None, trunc_values=None, bootstrap=None,
                       gamma=0.99, out=None):
    """Discounted returns (Monte-Carlo when bootstrap is None)."""
    shape, dev = _rollout_shape(rewards)
    r = _steps("rewards", rewards, shape, torch.float32, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev)
    g = _out(out, shape, dev)
    _check(lib().rlca_discounted_returns(_ptr(r), _ptr(term), _ptr(trunc), _ptr(tv), _ptr(boot),
                                         gamma, shape[0], shape[1], _ptr(g), _stream(r)),
           "rlca_discounted_returns")
    return g


def vtrace(rewards, values, behaviour_logp, target_logp, terminated, truncated=None,
           trunc_values=None, bootstrap=None, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0,
           with_pg=True, vs=None, pg_advantages=None):
    """V-Trace targets and policy-gradient advantages.  Returns (vs, pg|None)."""
    shape, dev = _rollout_shape(rewards)
    r = _steps("rewards", rewards, shape, torch.float32, dev)
    v = _steps("values", values, shape, torch.float32, dev)
    mu = _steps("behaviour_logp", behaviour_logp, shape, torch.float32, dev)
    pi = _steps("target_logp", target_logp, shape, torch.float32, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev)
    o_vs = _out(vs, shape, dev, name="vs")
    o_pg = _out(pg_advantages, shape, dev, name="pg_advantages") if with_pg else None
    _check(lib().rlca_vtrace(_ptr(r), _ptr(v), _ptr(mu), _ptr(pi), _ptr(term), _ptr(trunc),
                             _ptr(tv), _ptr(boot), gamma, lam, rho_bar, c_bar, shape[0],
                             shape[1], _ptr(o_vs), _ptr(o_pg), _stream(r)), "rlca_vtrace")
    return o_vs, o_pg


def retrace(rewards, q_values, expected_q, behaviour_logp, target_logp, terminated,
            truncated=None, trunc_values=None, bootstrap=None, gamma=0.99, lam=0.95,
            c_bar=1.0, out=None):
    """Retrace(lambda) targets Q^ret."""
    shape, dev = _rollout_shape(rewards)
    r = _steps("rewards", rewards, shape, torch.float32, dev)
    q = _steps("q_values", q_values, shape, torch.float32, dev)
    eq = _steps("expected_q", expected_q, shape, torch.float32, dev)
    mu = _steps("behaviour_logp", behaviour_logp, shape, torch.float32, dev)
    pi = _steps("target_logp", target_logp, shape, torch.float32, dev)
    term, trunc, tv, boot = _boundary(terminated, truncated, trunc_values, bootstrap, shape, dev)
    o = _out(out, shape, dev)
    _check(lib().rlca_retrace(_ptr(r), _ptr(q), _ptr(eq), _ptr(mu), _ptr(pi), _ptr(term),
                              _ptr(trunc), _ptr(tv), _ptr(boot), gamma, lam, c_bar, shape[0],
                              shape[1], _ptr(o), _stream(r)), "rlca_retrace")
    return o


def eligibility_traces(increments, flags, convention=RESET_ON_START, gamma=0.99, lam=0.9,
                       out=None):
    """Accumulating eligibility traces, forward in time."""
    shape, dev = _rollout_shape(increments)
    x = _steps("increments", increments, shape, torch.float32, dev)
    f = _steps("flags", flags, shape, "flag", dev)
    o = _out(out, shape, dev)
    _check(lib().rlca_eligibility_traces(_ptr(x), _ptr(f), int(convention), gamma, lam,
                                         shape[0], shape[1], _ptr(o), _stream(x)),
           "rlca_eligibility_traces")
    return o


def episodic_prefix_sum(x, flags, convention=RESET_ON_START, out=None):
    """Inclusive segmented prefix sum over float32 or int32 input (int32 wraps)."""
    shape, dev = _rollout_shape(x)
    if x.dtype == torch.float32:
        dtype = RLCA_F32
    elif x.dtype == torch.int32:
        dtype = RLCA_I32
    else:
        raise TypeError(f"x must be float32 or int32, got {x.dtype}")
    xs = _steps("x", x, shape, x.dtype, dev)
    f = _steps("flags", flags, shape, "flag", dev)
    o = _out(out, shape, dev, dtype=x.dtype)
    _check(lib().rlca_episodic_prefix_sum(_ptr(xs), dtype, _ptr(f), int(convention), shape[0],
                                          shape[1], _ptr(o), _stream(xs)),
           "rlca_episodic_prefix_sum")
    return o


def affine_scan(alpha, beta, carry=None, direction=BACKWARD, out=None):
    """A_t = alpha_t + beta_t * A_{t+1} (BACKWARD, A_T = carry) or
    A_t = alpha_t + beta_t * A_{t-1} (FORWARD, A_{-1} = carry), float32."""
    shape, dev = _rollout_shape(alpha)
    a = _steps("alpha", alpha, shape, torch.float32, dev)
    b = _steps("beta", beta, shape, torch.float32, dev)
    c = _steps("carry", carry, shape[:1], torch.float32, dev, optional=True)
    o = _out(out, shape, dev)
    _check(lib().rlca_affine_scan(_ptr(a), _ptr(b), _ptr(c), int(direction), shape[0], shape[1],
                                  _ptr(o), _stream(a)), "rlca_affine_scan")
    return o
