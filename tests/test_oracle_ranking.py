"""Pins for the ranking-quality oracle (CPU only).

oracle/ranking.py is checked against:
  * brute force: pure-Python loops over every budget with math.fsum and an
    explicit sort by (-score, position),
  * the rearrangement inequality: no order costs less than the order of the
    importance itself, the reversed order costs the most, and a uniform
    importance u costs u * n (n + 1) / 2 under every order,
  * the rank identity: the entry ranked r is evicted at the r + 1 budgets
    0 .. r, so the cost is sum_r (r + 1) * importance,
  * set arithmetic for the recall (equal, disjoint, brute-force overlap),
and each pin rejects a plausible mistake (a budget range that skips b = 0).
"""
import math

import numpy as np
import pytest

from oracle import ranking as rk


def brute_cost(scores, importance):
    n = len(scores)
    order = sorted(range(n), key=lambda j: (-scores[j], j))
    terms = []
    for b in range(n + 1):
        evicted = order[b:]
        terms.append(math.fsum(importance[j] for j in evicted))
    return math.fsum(terms)


@pytest.mark.parametrize("seed,n", [(0, 1), (1, 7), (2, 40), (3, 100)])
def test_cost_matches_brute_force(seed, n):
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal(n)
    scores[rng.random(n) < 0.2] = 0.5            # ties
    imp = rng.random(n) ** 3
    got = rk.eviction_cost(imp[None], rk.rank_order(scores[None]))[0]
    assert got == pytest.approx(brute_cost(scores.tolist(), imp.tolist()), rel=1e-13)
    # a budget range that skips b = 0 (where every entry is evicted) must differ
    if n > 1 and imp.sum() > 0:
        order = rk.rank_order(scores[None])[0]
        ranked = imp[order]
        wrong = np.sum(ranked.sum() - np.cumsum(ranked))             # b = 1 .. n only
        assert not math.isclose(wrong, got, rel_tol=1e-9)


def test_rank_identity_and_rearrangement():
    rng = np.random.default_rng(5)
    H, n = 4, 300
    imp = rng.random((H, n)) ** 2
    opt = rk.eviction_cost(imp, rk.rank_order(imp))
    worst = rk.eviction_cost(imp, rk.rank_order(-imp))
    for h in range(H):
        desc = np.sort(imp[h])[::-1]
        assert opt[h] == pytest.approx(np.sum(np.arange(1, n + 1) * desc), rel=1e-13)
        assert worst[h] == pytest.approx(np.sum(np.arange(n, 0, -1) * desc), rel=1e-13)
    for seed in range(5):
        s = np.random.default_rng(100 + seed).standard_normal((H, n))
        c = rk.eviction_cost(imp, rk.rank_order(s))
        assert np.all(c >= opt * (1 - 1e-14)) and np.all(c <= worst * (1 + 1e-14))
    np.testing.assert_allclose(rk.normalized_cost(imp, imp), 1.0, rtol=0, atol=0)


def test_uniform_importance_costs_the_same_under_every_order():
    n, u = 77, 0.25
    imp = np.full((1, n), u)
    for seed in range(4):
        s = np.random.default_rng(seed).standard_normal((1, n))
        assert rk.eviction_cost(imp, rk.rank_order(s))[0] == pytest.approx(u * n * (n + 1) / 2, rel=1e-14)
        assert rk.normalized_cost(s, imp)[0] == pytest.approx(1.0, rel=1e-14)   # every order is optimal


def test_normalised_cost_without_importance_is_one():
    """No importance at all: both costs are 0 and the ratio is read as 1
    (every ranking evicts nothing at every budget); one head with and one
    without importance keep their own ratios."""
    s = np.random.default_rng(5).standard_normal((2, 40))
    imp = np.zeros((2, 40))
    imp[1, 7] = 1.0                                     # head 1: one entry carries everything
    r = rk.normalized_cost(s, imp)
    assert r[0] == 1.0
    pos = int(np.where(rk.rank_order(s[1:])[0] == 7)[0][0])
    assert r[1] == pytest.approx((pos + 1) / 1.0, rel=1e-14)   # evicted at budgets 0 .. pos


def test_rank_order_ties_nan_and_signed_zero():
    s = np.array([[0.0, -0.0, np.nan, 1.0, np.inf, -np.inf, 1.0, np.nan]])
    assert rk.rank_order(s)[0].tolist() == [4, 3, 6, 0, 1, 5, 2, 7]


def test_retention_recall_sets():
    assert rk.retention_recall([1, 2, 3], [3, 2, 1]) == 1.0
    assert rk.retention_recall([1, 2, 3], [4, 5]) == 0.0
    rng = np.random.default_rng(3)
    a = rng.choice(1000, 200, replace=False)
    b = rng.choice(1000, 300, replace=False)
    assert rk.retention_recall(a, b) == len([x for x in a if x in set(b.tolist())]) / 200
    assert rk.retention_recall([5, 5, 6], [5, 7]) == 0.5       # duplicates count once
