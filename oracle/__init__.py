"""Plain sequential fp64 CPU oracle for the seven credit-assignment estimators.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(the HIP library and its Python binding) never does, and this package imports
nothing from it.  The arithmetic lives in ``oracle.c`` (plain C99, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays.

Definitions follow "rl-triton: High-Performance Triton GPU Kernels for
Reinforcement Learning Credit Assignment" (paperlayer.ai summary), §1, §2.1,
§3.2, §3.3, §5 and §8; the header of ``oracle.c`` states the boundary rules.

The fused consumers (``mean_std``, ``ppo_clip_loss``) follow the standard
advantage normalization and the PPO clipped surrogate of Schulman et al. 2017;
the summary's §9 names fused loss operations as the next step.

Pins (tests/test_oracle_pins.py): brute-force unrolled sums on tiny inputs,
products-of-coefficients sums for the generic affine scan,
closed forms, the cross-estimator identities (GAE lambda=0 / lambda=1,
V-Trace on-policy, Retrace lambda=0), no-leak invariance at done steps and the
worked four-thread trace of the summary's Appendix A.  Every function here is
pinned by at least one of them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

RESET_ON_START = 0
RESET_AFTER_DONE = 1
BACKWARD = 0
FORWARD = 1

_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_dbl = ctypes.c_double


def _load():
    global _lib
    if _lib is None:
        # RLCA_ORACLE_LIB names another build of oracle.c to load instead; the
        # mutation test points it at builds with a planted mistake.
        path = os.environ.get("RLCA_ORACLE_LIB")
        if path is None:
            path = LIB_PATH
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        sig = {
            "oracle_gae": [_f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _dbl, _dbl, _i64, _i64,
                           _f64p, _f64p],
            "oracle_td_lambda": [_f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _dbl, _dbl, _i64,
                                 _i64, _f64p],
            "oracle_discounted_returns": [_f32p, _u8p, _u8p, _f32p, _f32p, _dbl, _i64, _i64,
                                          _f64p],
            "oracle_vtrace": [_f32p, _f32p, _f32p, _f32p, _u8p, _u8p, _f32p, _f32p, _dbl,
                              _dbl, _dbl, _dbl, _i64, _i64, _f64p, _f64p],
            "oracle_retrace": [_f32p, _f32p, _f32p, _f32p, _f32p, _u8p, _u8p, _f32p, _f32p,
                               _dbl, _dbl, _dbl, _i64, _i64, _f64p],
            "oracle_eligibility_traces": [_f32p, _u8p, ctypes.c_int, _dbl, _dbl, _i64, _i64,
                                          _f64p],
            "oracle_episodic_prefix_sum_f32": [_f32p, _u8p, ctypes.c_int, _i64, _i64, _f64p],
            "oracle_episodic_prefix_sum_i32": [_i32p, _u8p, ctypes.c_int, _i64, _i64, _i32p],
            "oracle_affine_scan": [_f32p, _f32p, _f32p, ctypes.c_int, _i64, _i64, _f64p],
            "oracle_mean_std": [_f64p, _i64, _f64p, _f64p],
            "oracle_ppo_clip_loss": [_f32p, _f32p, _f32p, _i64, ctypes.c_int, _dbl, _dbl, _dbl,
                                     _dbl, _f64p, _f64p],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        _lib = lib
    return _lib


def _arr(x, dtype, shape):
    """Contiguous copy-free view of ``x`` as ``dtype``; None stays None."""
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=dtype)
    if a.shape != shape:
        raise ValueError(f"expected shape {shape}, got {a.shape}")
    ptype = {np.float32: _f32p, np.uint8: _u8p, np.int32: _i32p, np.float64: _f64p}[dtype]
    return a, a.ctypes.data_as(ptype)


def _flags(x, shape):
    if x is None:
        return _arr(None, np.uint8, shape)
    return _arr((np.asarray(x) != 0).astype(np.uint8), np.uint8, shape)


def _shape(rewards):
    r = np.asarray(rewards)
    if r.ndim != 2:
        raise ValueError("per-step inputs are [num_envs, T]")
    return r.shape


def _trunc_args(truncated, trunc_values, shape):
    trunc, trunc_p = _flags(truncated, shape)
    tv, tv_p = _arr(trunc_values, np.float32, shape)
    if trunc is not None and tv is None:
        raise ValueError("trunc_values is required when truncated is given")
    return trunc, trunc_p, tv, tv_p


def gae(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
        gamma=0.99, lam=0.95):
    """Generalized advantage estimation.  Returns (advantages, returns), float64."""
    shape = _shape(rewards)
    n, t = shape
    r, rp = _arr(rewards, np.float32, shape)
    v, vp = _arr(values, np.float32, shape)
    d, dp = _flags(terminated, shape)
    tr, trp, tv, tvp = _trunc_args(truncated, trunc_values, shape)
    b, bp = _arr(bootstrap, np.float32, (n,))
    adv = np.empty(shape, np.float64)
    ret = np.empty(shape, np.float64)
    _load().oracle_gae(rp, vp, dp, trp, tvp, bp, gamma, lam, n, t,
                       adv.ctypes.data_as(_f64p), ret.ctypes.data_as(_f64p))
    return adv, ret


def td_lambda(rewards, values, terminated, truncated=None, trunc_values=None, bootstrap=None,
              gamma=0.99, lam=0.95):
    """TD(lambda) returns, float64."""
    shape = _shape(rewards)
    n, t = shape
    r, rp = _arr(rewards, np.float32, shape)
    v, vp = _arr(values, np.float32, shape)
    d, dp = _flags(terminated, shape)
    tr, trp, tv, tvp = _trunc_args(truncated, trunc_values, shape)
    b, bp = _arr(bootstrap, np.float32, (n,))
    out = np.empty(shape, np.float64)
    _load().oracle_td_lambda(rp, vp, dp, trp, tvp, bp, gamma, lam, n, t,
                             out.ctypes.data_as(_f64p))
    return out


def discounted_returns(rewards, terminated, truncated=None, trunc_values=None, bootstrap=None,
                       gamma=0.99):
    """Discounted returns, float64."""
    shape = _shape(rewards)
    n, t = shape
    r, rp = _arr(rewards, np.float32, shape)
    d, dp = _flags(terminated, shape)
    tr, trp, tv, tvp = _trunc_args(truncated, trunc_values, shape)
    b, bp = _arr(bootstrap, np.float32, (n,))
    out = np.empty(shape, np.float64)
    _load().oracle_discounted_returns(rp, dp, trp, tvp, bp, gamma, n, t,
                                      out.ctypes.data_as(_f64p))
    return out


def vtrace(rewards, values, behaviour_logp, target_logp, terminated, truncated=None,
           trunc_values=None, bootstrap=None, gamma=0.99, lam=1.0, rho_bar=1.0, c_bar=1.0):
    """V-Trace targets and policy-gradient advantages.  Returns (vs, pg), float64."""
    shape = _shape(rewards)
    n, t = shape
    r, rp = _arr(rewards, np.float32, shape)
    v, vp = _arr(values, np.float32, shape)
    mu, mup = _arr(behaviour_logp, np.float32, shape)
    pi, pip = _arr(target_logp, np.float32, shape)
    d, dp = _flags(terminated, shape)
    tr, trp, tv, tvp = _trunc_args(truncated, trunc_values, shape)
    b, bp = _arr(bootstrap, np.float32, (n,))
    vs = np.empty(shape, np.float64)
    pg = np.empty(shape, np.float64)
    _load().oracle_vtrace(rp, vp, mup, pip, dp, trp, tvp, bp, gamma, lam, rho_bar, c_bar,
                          n, t, vs.ctypes.data_as(_f64p), pg.ctypes.data_as(_f64p))
    return vs, pg


def retrace(rewards, q_values, expected_q, behaviour_logp, target_logp, terminated,
            truncated=None, trunc_values=None, bootstrap=None, gamma=0.99, lam=0.95,
            c_bar=1.0):
    """Retrace(lambda) targets Q^ret, float64."""
    shape = _shape(rewards)
    n, t = shape
    r, rp = _arr(rewards, np.float32, shape)
    q, qp = _arr(q_values, np.float32, shape)
    eq, eqp = _arr(expected_q, np.float32, shape)
    mu, mup = _arr(behaviour_logp, np.float32, shape)
    pi, pip = _arr(target_logp, np.float32, shape)
    d, dp = _flags(terminated, shape)
    tr, trp, tv, tvp = _trunc_args(truncated, trunc_values, shape)
    b, bp = _arr(bootstrap, np.float32, (n,))
    out = np.empty(shape, np.float64)
    _load().oracle_retrace(rp, qp, eqp, mup, pip, dp, trp, tvp, bp, gamma, lam, c_bar, n, t,
                           out.ctypes.data_as(_f64p))
    return out


def eligibility_traces(increments, flags, convention=RESET_ON_START, gamma=0.99, lam=0.9):
    """Accumulating eligibility traces (forward scan), float64."""
    shape = _shape(increments)
    n, t = shape
    x, xp = _arr(increments, np.float32, shape)
    f, fp = _flags(flags, shape)
    out = np.empty(shape, np.float64)
    _load().oracle_eligibility_traces(xp, fp, int(convention), gamma, lam, n, t,
                                      out.ctypes.data_as(_f64p))
    return out


def episodic_prefix_sum(x, flags, convention=RESET_ON_START):
    """Inclusive segmented prefix sum.  float32 input -> float64 output;
    int32 input -> int32 output with two's-complement wrap-around."""
    shape = _shape(x)
    n, t = shape
    f, fp = _flags(flags, shape)
    xa = np.asarray(x)
    if xa.dtype == np.int32:
        xi, xip = _arr(xa, np.int32, shape)
        out = np.empty(shape, np.int32)
        _load().oracle_episodic_prefix_sum_i32(xip, fp, int(convention), n, t,
                                               out.ctypes.data_as(_i32p))
        return out
    if xa.dtype != np.float32:
        raise TypeError("episodic_prefix_sum takes float32 or int32 input")
    xf, xfp = _arr(xa, np.float32, shape)
    out = np.empty(shape, np.float64)
    _load().oracle_episodic_prefix_sum_f32(xfp, fp, int(convention), n, t,
                                           out.ctypes.data_as(_f64p))
    return out


def affine_scan(alpha, beta, carry=None, direction=BACKWARD):
    """A_t = alpha_t + beta_t * A_{t+1} (BACKWARD, A_T = carry) or
    A_t = alpha_t + beta_t * A_{t-1} (FORWARD, A_{-1} = carry), float64."""
    shape = _shape(alpha)
    n, t = shape
    a, ap = _arr(alpha, np.float32, shape)
    b, bp = _arr(beta, np.float32, shape)
    c, cp = _arr(carry, np.float32, (n,))
    out = np.empty(shape, np.float64)
    _load().oracle_affine_scan(ap, bp, cp, int(direction), n, t, out.ctypes.data_as(_f64p))
    return out


def mean_std(x):
    """(mean, sample std with divisor M - 1) of all elements of x, in fp64."""
    a = np.ascontiguousarray(np.asarray(x, np.float64).ravel())
    mean, std = ctypes.c_double(), ctypes.c_double()
    _load().oracle_mean_std(a.ctypes.data_as(_f64p), a.size, ctypes.byref(mean),
                            ctypes.byref(std))
    return mean.value, std.value


def ppo_clip_loss(adv, logp_new, logp_old, stats=None, clip_eps=0.2, norm_eps=1e-8):
    """PPO clipped-surrogate loss and its gradient w.r.t. logp_new, float64.
    stats = (mean, std) normalizes the advantages first; None uses them raw."""
    a = np.ascontiguousarray(np.asarray(adv, np.float32).ravel())
    shape = np.asarray(adv).shape
    new, newp = _arr(np.asarray(logp_new, np.float32).ravel(), np.float32, a.shape)
    old, oldp = _arr(np.asarray(logp_old, np.float32).ravel(), np.float32, a.shape)
    mean, std = stats if stats is not None else (0.0, 1.0)
    loss = ctypes.c_double()
    grad = np.empty(a.shape, np.float64)
    _load().oracle_ppo_clip_loss(a.ctypes.data_as(_f32p), newp, oldp, a.size,
                                 1 if stats is not None else 0, mean, std, norm_eps, clip_eps,
                                 ctypes.byref(loss), grad.ctypes.data_as(_f64p))
    return loss.value, grad.reshape(shape)
