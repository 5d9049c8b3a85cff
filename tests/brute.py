"""Brute-force closed-sum forms of the seven estimators, in Python floats.

These pin the oracle: each estimator is written here as the explicit sum over
the rest of its episode segment (the unrolled form of the recursion), not as a
recursion, so a dropped term, a wrong exponent or a wrong index in the oracle's
one-step updates shows up as a mismatch.  Quadratic or worse in T: tiny inputs
only.

Boundary rules (rl-triton, paperlayer.ai summary §3.2): a terminated step has
successor value 0, a truncated step (terminated wins) uses the supplied
continuation value, and the window's last step uses the row's bootstrap; all
three end the segment.  Forward resets: §3.3 and §5.
"""
from __future__ import annotations

import math

import numpy as np


def _f(x):
    return float(x)


class Row:
    """One row of a rollout with its segment structure."""

    def __init__(self, T, term, trunc=None, tv=None, b=0.0):
        self.T = T
        self.term = [bool(x) for x in term]
        self.trunc = [bool(x) and not self.term[i]
                      for i, x in enumerate(trunc if trunc is not None else [0] * T)]
        self.tv = [_f(x) for x in (tv if tv is not None else [0.0] * T)]
        self.b = _f(b)

    def stops(self, j):
        return self.term[j] or self.trunc[j] or j == self.T - 1

    def seg_end(self, t):
        j = t
        while not self.stops(j):
            j += 1
        return j

    def succ(self, j):
        """Successor value at a step that ends its segment."""
        if self.term[j]:
            return 0.0
        if self.trunc[j]:
            return self.tv[j]
        return self.b


def _rows(N, T, term, trunc, tv, b):
    out = []
    for n in range(N):
        out.append(Row(T, term[n], None if trunc is None else trunc[n],
                       None if tv is None else tv[n], 0.0 if b is None else b[n]))
    return out


def gae(r, v, term, trunc, tv, b, gamma, lam):
    N, T = r.shape
    adv = np.zeros((N, T))
    for n, row in enumerate(_rows(N, T, term, trunc, tv, b)):
        for t in range(T):
            e = row.seg_end(t)
            s = 0.0
            for j in range(t, e + 1):
                nxt = _f(v[n, j + 1]) if j < e else row.succ(e)
                delta = _f(r[n, j]) + gamma * nxt - _f(v[n, j])
                s += (gamma * lam) ** (j - t) * delta
            adv[n, t] = s
    return adv, adv + v.astype(np.float64)


def discounted(r, term, trunc, tv, b, gamma):
    N, T = r.shape
    out = np.zeros((N, T))
    for n, row in enumerate(_rows(N, T, term, trunc, tv, b)):
        for t in range(T):
            e = row.seg_end(t)
            s = sum(gamma ** (j - t) * _f(r[n, j]) for j in range(t, e + 1))
            out[n, t] = s + gamma ** (e - t + 1) * row.succ(e)
    return out


def td_lambda(r, v, term, trunc, tv, b, gamma, lam):
    """Forward view: lambda-weighted mixture of n-step returns, truncated at the
    segment end where the full (Monte-Carlo plus successor) return takes the
    remaining weight lambda^(e-t)."""
    N, T = r.shape
    out = np.zeros((N, T))
    for n, row in enumerate(_rows(N, T, term, trunc, tv, b)):
        for t in range(T):
            e = row.seg_end(t)
            full = sum(gamma ** (j - t) * _f(r[n, j]) for j in range(t, e + 1)) \
                + gamma ** (e - t + 1) * row.succ(e)
            g = lam ** (e - t) * full
            for k in range(1, e - t + 1):
                g_k = sum(gamma ** (j - t) * _f(r[n, j]) for j in range(t, t + k)) \
                    + gamma ** k * _f(v[n, t + k])
                g += (1.0 - lam) * lam ** (k - 1) * g_k
            out[n, t] = g
    return out


def _ratio(tl, bl, clip=5.0):
    lr = _f(tl) - _f(bl)
    return math.exp(min(clip, max(-clip, lr)))


def vtrace(r, v, blogp, tlogp, term, trunc, tv, b, gamma, lam, rho_bar, c_bar):
    """IMPALA n-step form: vs_t = V_t + sum_j gamma^(j-t) (prod_{i=t}^{j-1} c_i) delta_j."""
    N, T = r.shape
    vs = np.zeros((N, T))
    pg = np.zeros((N, T))
    for n, row in enumerate(_rows(N, T, term, trunc, tv, b)):
        ratio = [_ratio(tlogp[n, t], blogp[n, t]) for t in range(T)]
        rho = [min(rho_bar, x) for x in ratio]
        c = [lam * min(c_bar, x) for x in ratio]
        for t in range(T):
            e = row.seg_end(t)
            s = _f(v[n, t])
            for j in range(t, e + 1):
                nxt = _f(v[n, j + 1]) if j < e else row.succ(e)
                delta = rho[j] * (_f(r[n, j]) + gamma * nxt - _f(v[n, j]))
                s += gamma ** (j - t) * math.prod(c[t:j]) * delta
            vs[n, t] = s
        for t in range(T):
            nxt = vs[n, t + 1] if not row.stops(t) else row.succ(t)
            pg[n, t] = rho[t] * (_f(r[n, t]) + gamma * nxt - _f(v[n, t]))
    return vs, pg


def retrace(r, q, eq, blogp, tlogp, term, trunc, tv, b, gamma, lam, c_bar):
    """Munos et al. sum: Qret_t = Q_t + sum_j gamma^(j-t) (prod_{i=t+1}^{j} c_i) delta_j,
    delta_j = r_j + gamma E_pi Q(s_{j+1}) - Q_j."""
    N, T = r.shape
    out = np.zeros((N, T))
    for n, row in enumerate(_rows(N, T, term, trunc, tv, b)):
        c = [lam * min(c_bar, _ratio(tlogp[n, t], blogp[n, t])) for t in range(T)]
        for t in range(T):
            e = row.seg_end(t)
            s = _f(q[n, t])
            for j in range(t, e + 1):
                nxt = _f(eq[n, j + 1]) if j < e else row.succ(e)
                delta = _f(r[n, j]) + gamma * nxt - _f(q[n, j])
                s += gamma ** (j - t) * math.prod(c[t + 1:j + 1]) * delta
            out[n, t] = s
    return out


def _segment_start(flags_row, convention, t):
    s = 0
    for j in range(1, t + 1):
        if (convention == 0 and flags_row[j]) or (convention == 1 and flags_row[j - 1]):
            s = j
    return s


def eligibility(x, flags, convention, gamma, lam):
    N, T = x.shape
    out = np.zeros((N, T))
    for n in range(N):
        for t in range(T):
            s = _segment_start(flags[n], convention, t)
            out[n, t] = sum((gamma * lam) ** (t - j) * _f(x[n, j]) for j in range(s, t + 1))
    return out


def prefix_sum(x, flags, convention):
    """Per-segment numpy cumsum (int64 for integers, then wrapped to int32)."""
    N, T = x.shape
    is_int = np.issubdtype(x.dtype, np.integer)
    out = np.zeros((N, T), np.int64 if is_int else np.float64)
    for n in range(N):
        starts = [t for t in range(T) if _segment_start(flags[n], convention, t) == t]
        bounds = starts + [T]
        for a, z in zip(bounds[:-1], bounds[1:]):
            seg = x[n, a:z].astype(np.int64 if is_int else np.float64)
            out[n, a:z] = np.cumsum(seg)
    if is_int:
        return out.astype(np.uint64).astype(np.uint32).view(np.int32)
    return out


def affine(alpha, beta, carry, direction):
    """Unrolled: backward A_t = sum_{j>=t} (prod_{i=t}^{j-1} beta_i) alpha_j
    + (prod_{i=t}^{T-1} beta_i) carry; forward mirrored."""
    N, T = alpha.shape
    out = np.zeros((N, T))
    for n in range(N):
        c = 0.0 if carry is None else _f(carry[n])
        for t in range(T):
            js = range(t, T) if direction == 0 else range(t, -1, -1)
            s = 0.0
            for j in js:
                span = range(t, j) if direction == 0 else range(j + 1, t + 1)
                s += math.prod(_f(beta[n, i]) for i in span) * _f(alpha[n, j])
            whole = range(t, T) if direction == 0 else range(0, t + 1)
            s += math.prod(_f(beta[n, i]) for i in whole) * c
            out[n, t] = s
    return out
