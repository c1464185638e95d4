"""Closed-form Soft-TopK and learned per-head budgets (LKV), fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

LKV, "The Differentiable Soft-TopK Operator", states three properties of
ST_k (its output sums to k, it preserves order, it is invariant to adding a
constant) and prints only the threshold

    lambda = log( (sqrt((k-m)^2 + S1*S2) - (k-m)) / S1 ),
    S1 = sum_{i<=m} exp(-x_i),  S2 = sum_{i>m} exp(x_i),

with x sorted in decreasing order. The mask itself and m are not printed.
The reading used here: the mask is the Laplace CDF of (x_i - lambda)/tau,

    mask_i = 1 - exp(-(x_i - lambda)) / 2   if x_i >= lambda,
    mask_i =     exp(  x_i - lambda ) / 2   otherwise,

and m is the number of entries at or above lambda. Requiring the masks to sum
to k gives m - e^lambda S1 / 2 + e^-lambda S2 / 2 = k, a quadratic in
e^lambda whose positive root is exactly the printed threshold. The sum is
strictly decreasing in lambda, so exactly one m is self-consistent.

LKV, "LKV-H: Learning Global Budget Allocation": retention ratios are the
Soft-TopK of the flattened head scores with k = R_agg (so they sum to
R_agg), frozen, and the budget of head (l, h) at length t is floor(r * t).
LKV, "Theoretical and Practical Implications": at k = 1 the operator
approximates softmax, and it tends to hard top-k as tau -> 0.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def _logsumexp(v: np.ndarray) -> float:
    if v.size == 0:
        return -math.inf
    top = float(v.max())
    return top + math.log(float(np.exp(v - top).sum()))


def _logaddexp(a: float, b: float) -> float:
    return float(np.logaddexp(a, b))


def threshold(x: np.ndarray, k: float, tau: float = 1.0) -> Tuple[float, int]:
    """Return (lambda on the x/tau scale, m) for ``0 < k < len(x)``."""
    z = np.sort(np.asarray(x, dtype=np.float64) / tau)[::-1]
    n = z.size
    if not 0.0 < k < n:
        raise ValueError("need 0 < k < n")
    for m in range(n + 1):
        log_s1 = _logsumexp(-z[:m])
        log_s2 = _logsumexp(z[m:])
        a = k - m
        if m == 0:
            lam = log_s2 - math.log(2.0 * k)                 # S1 = 0 limit
        elif m == n:
            lam = math.log(2.0 * (n - k)) - log_s1            # S2 = 0 limit
        else:
            log_p = log_s1 + log_s2                           # log(S1*S2)
            if a > 0:
                # e^lambda = S2 / (sqrt(a^2 + P) + a): no cancellation
                root = 0.5 * _logaddexp(2.0 * math.log(a), log_p)
                lam = log_s2 - _logaddexp(root, math.log(a))
            elif a < 0:
                root = 0.5 * _logaddexp(2.0 * math.log(-a), log_p)
                lam = _logaddexp(root, math.log(-a)) - log_s1
            else:
                lam = 0.5 * log_p - log_s1
        upper_ok = m == 0 or z[m - 1] >= lam
        lower_ok = m == n or lam > z[m]
        if upper_ok and lower_ok:
            return lam, m
    raise RuntimeError("no self-consistent m (non-finite input?)")


def laplace_mask(z: np.ndarray, lam: float) -> np.ndarray:
    """Laplace CDF of ``z - lam``."""
    u = z - lam
    out = np.empty_like(u)
    hi = u >= 0
    out[hi] = 1.0 - 0.5 * np.exp(-u[hi])
    out[~hi] = 0.5 * np.exp(u[~hi])
    return out


def soft_topk(x: np.ndarray, k: float, tau: float = 1.0) -> np.ndarray:
    """ST_k(x; tau): entries in (0, 1), summing to k, in the input order."""
    x = np.asarray(x, dtype=np.float64)
    lam, _ = threshold(x, k, tau)
    return laplace_mask(x / tau, lam)


def head_ratios(head_scores: np.ndarray, mean_ratio: float, tau: float = 1.0) -> np.ndarray:
    """Retention ratios of all L*H heads, summing to ``R_agg = mean * L*H``."""
    s = np.asarray(head_scores, dtype=np.float64).ravel()
    return soft_topk(s, mean_ratio * s.size, tau).reshape(np.shape(head_scores))


def head_budgets(ratios: np.ndarray, t: int) -> np.ndarray:
    """``floor(r * t)`` per head."""
    return np.floor(np.asarray(ratios, dtype=np.float64) * t).astype(np.int64)
