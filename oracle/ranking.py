"""Ranking-quality measures (fp64 / numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages:

* KVP, section 3: the top-b entries of a per-head ranking form the cache for
  any budget b, so eviction reduces to ranking.
* KVP, 3.1.1 (the global reward): a ranking is judged by the future-attention
  importance of the entries it evicts, accumulated over the cache budgets as
  a cost-versus-budget area under the curve, and normalised by the cost of the
  optimal ranking.
* KVpop, Figure 7: top-k retention recall, the fraction of the full-attention
  teacher's retained tokens that another scorer also retains under the same
  budget.

Readings where the pages are silent: the budgets are every b = 0 .. n (keep
the b best entries, evict the rest); the cost at a budget is the summed
importance of the evicted entries; the area is the plain sum over budgets;
normalising divides by the area of the ranking by importance itself (so 1 is
optimal and larger is worse), and is 1 when there is no importance to
evict at all (both costs 0); rankings order by score descending with ties
to the lower position, NaN last, -0.0 equal to +0.0 (as in selection); the
recall divides the overlap by the size of the teacher's kept set.
"""
from __future__ import annotations

import numpy as np

from .select_oracle import rank_candidates


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Per row, the positions of the entries best first: ``[H, n]`` int64."""
    scores = np.atleast_2d(scores)
    n = scores.shape[1]
    return np.stack([rank_candidates(row, np.arange(n)) for row in scores])


def eviction_cost(importance: np.ndarray, order: np.ndarray) -> np.ndarray:
    """Sum over budgets b = 0 .. n of the importance the order evicts at b.

    At budget b the first b positions of ``order`` stay and the rest are
    evicted. Returns ``[H]`` fp64.
    """
    importance = np.atleast_2d(np.asarray(importance, dtype=np.float64))
    order = np.atleast_2d(order)
    H, n = importance.shape
    out = np.empty(H, dtype=np.float64)
    for h in range(H):
        ranked = importance[h][order[h]]
        kept = np.concatenate([[0.0], np.cumsum(ranked)])   # importance kept at b = 0 .. n
        out[h] = np.sum(ranked.sum() - kept)
    return out


def normalized_cost(scores: np.ndarray, importance: np.ndarray) -> np.ndarray:
    """Cost of ranking by ``scores`` over the cost of ranking by ``importance``.

    Where the optimal cost is 0 and so is the ranking's cost (no importance
    to evict at any budget), every ranking is optimal and the ratio is 1;
    otherwise the ratio is the plain quotient.
    """
    c = eviction_cost(importance, rank_order(scores))
    c_opt = eviction_cost(importance, rank_order(importance))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = c / c_opt
    ratio[(c == 0.0) & (c_opt == 0.0)] = 1.0
    return ratio


def retention_recall(kept_teacher, kept_other) -> float:
    """|teacher's kept set & other's kept set| / |teacher's kept set|."""
    a, b = set(np.asarray(kept_teacher).tolist()), set(np.asarray(kept_other).tolist())
    return len(a & b) / len(a) if a else 1.0
