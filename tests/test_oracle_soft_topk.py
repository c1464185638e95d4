"""Pins for the Soft-TopK oracle and the KVpop target epilogue (CPU only).

Soft-TopK: the three properties the LKV page states (sum to k, order
preserving, translation invariant), an independent bisection of the
threshold on the mask definition, the printed closed form evaluated
literally, the softmax reduction at k = 1 and hard top-k as tau -> 0.
KVpop target: the page's worked example (tests/golden/kvpop_worked_example.json).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import kvpop_target as kt
from oracle import soft_topk as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bisect_lambda(z, k):
    """Solve sum(laplace(z - lam)) = k by bisection (independent of the closed form)."""
    def total(lam):
        u = z - lam
        return float(np.where(u >= 0, 1 - 0.5 * np.exp(-np.abs(u)), 0.5 * np.exp(-np.abs(u))).sum())
    lo, hi = z.min() - 60.0, z.max() + 60.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) > k:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


@pytest.mark.parametrize("seed,n,k,tau", [(0, 10, 3.0, 1.0), (1, 50, 7.5, 0.7), (2, 224, 33.6, 2.0),
                                          (3, 5, 4.9, 1.0), (4, 30, 0.2, 1.0), (5, 64, 1.0, 0.3)])
def test_properties_and_bisection(seed, n, k, tau):
    x = np.random.default_rng(seed).standard_normal(n) * 2.0
    m = st.soft_topk(x, k, tau)
    assert np.all((m > 0) & (m < 1))
    assert m.sum() == pytest.approx(k, rel=1e-12)
    order = np.argsort(x)
    assert np.all(np.diff(m[order]) >= 0)                                  # order preserving
    np.testing.assert_allclose(st.soft_topk(x + 3.25, k, tau), m, rtol=1e-10)  # translation
    lam, _ = st.threshold(x, k, tau)
    assert lam == pytest.approx(bisect_lambda(x / tau, k), abs=1e-9)


@pytest.mark.parametrize("seed", range(5))
def test_printed_closed_form_literally(seed):
    x = np.random.default_rng(10 + seed).standard_normal(12)
    k = 4.3
    lam, m = st.threshold(x, k)
    z = np.sort(x)[::-1]
    if 0 < m < z.size:
        s1 = np.exp(-z[:m]).sum()
        s2 = np.exp(z[m:]).sum()
        printed = math.log((math.sqrt((k - m) ** 2 + s1 * s2) - (k - m)) / s1)
        assert lam == pytest.approx(printed, abs=1e-12)


def test_k1_is_softmax_when_no_entry_dominates():
    x = np.random.default_rng(7).standard_normal(40) * 0.5
    p = np.exp(x - x.max())
    p /= p.sum()
    assert p.max() < 0.5
    np.testing.assert_allclose(st.soft_topk(x, 1.0), p, rtol=1e-12)


def test_small_tau_is_hard_topk():
    x = np.random.default_rng(8).standard_normal(100)
    m = st.soft_topk(x, 10, tau=1e-4)
    top = np.argsort(-x)[:10]
    hard = np.zeros(100)
    hard[top] = 1.0
    np.testing.assert_allclose(m, hard, atol=1e-6)


def test_head_budgets_sum_and_floor():
    s = np.random.default_rng(9).standard_normal((28, 4))
    r = st.head_ratios(s, 0.15)
    assert r.shape == (28, 4)
    assert r.sum() == pytest.approx(0.15 * 112, rel=1e-12)
    b = st.head_budgets(r, 200000)
    assert np.all(b == np.floor(r * 200000)) and np.all(b <= 200000)


def test_kvpop_worked_example():
    with open(os.path.join(GOLDEN, "kvpop_worked_example.json")) as f:
        ex = json.load(f)
    S, t, w = ex["S"], ex["t"], ex["w"]
    assert kt.future_counts(S, w)[t] == ex["N_t"]
    per_q = np.zeros((2, S))
    per_q[:, t] = [sum(p) for p in ex["future_probabilities_per_query_head"]]
    mean = per_q[:, t] / kt.future_counts(S, w)[t]
    np.testing.assert_allclose(mean, ex["mean_mass_per_query_head"], atol=1e-12)
    dec = ex["printed_decimals"]
    np.testing.assert_allclose(np.round(np.log(mean), dec), ex["log_mean_mass_per_query_head"], atol=0)
    r = kt.target(per_q, w, eps=0.0, aggregate="max")
    assert round(r[t], dec) == ex["target_max_aggregate"]
    # probability-space mean aggregation
    assert kt.target(per_q, w, aggregate="mean")[t] == pytest.approx(math.log(0.175), abs=1e-12)


def test_kvpop_counts_floor_at_one():
    n = kt.future_counts(10, 3)
    assert n.tolist() == [7, 6, 5, 4, 3, 2, 1, 1, 1, 1]
