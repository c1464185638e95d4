"""Running top-k cut-off over static ranks (numpy / pure Python).

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages (KVpop, "Delayed Memory Scoring", "Efficient Online Pruning"
and Algorithm 2, "Running top-k cutoff computation for one KV head"):

* every token carries a static rank from a pre-sort by a priority score
  (rank 1 is the best);
* the budget is (s, w, k): s sink tokens, a protected window of w recent
  tokens, and k long-range tokens;
* every cut-off starts at -1; at query q the token t = q - w leaves the
  window, and it enters the eligible set E(q) only if t >= s (sinks are
  kept by the mask on their own and never compete);
* once |E(q)| >= k, tau_q is the rank the tree's prefix-count search returns
  for k, i.e. the smallest rank r such that at least k eligible tokens have
  a rank <= r: the rank of the k-th best eligible token;
* the sparse attention of query q keeps the sinks, the window and the
  eligible tokens with rank <= tau_q.

The page keeps E(q) in a Fenwick tree and searches it by binary lifting;
the value is an order statistic of E(q), so the oracle keeps E(q) as a
sorted list and reads its k-th entry.

Readings where the pages are silent or at odds:
* ranks order the static scores descending, ties to the lower position,
  NaN last (as selection does);
* k = 0: the smallest rank with at least 0 eligible tokens at or below it is
  0, so tau_q = 0 for every q and no eligible token passes;
* with fewer than k eligible tokens tau_q stays -1 as the algorithm leaves
  it, and the mask applies its predicate as printed: rank <= -1 holds for no
  token, so such a query keeps only the sinks and the window (the page's
  prose, "the top-k eligible tokens", would keep all of them instead; the
  printed predicate is followed).
"""
from __future__ import annotations

import bisect

import numpy as np

from .select_oracle import rank_candidates


def ranks_from_scores(scores: np.ndarray) -> np.ndarray:
    """Static rank (1 = best) of every position of one head."""
    n = scores.shape[0]
    order = rank_candidates(scores, np.arange(n))
    ranks = np.empty(n, dtype=np.int64)
    ranks[order] = np.arange(1, n + 1)
    return ranks


def cutoffs(ranks: np.ndarray, s: int, w: int, k: int) -> np.ndarray:
    """tau_0 .. tau_{S-1} of one head for the budget (s, w, k)."""
    S = ranks.shape[0]
    tau = np.full(S, -1, dtype=np.int64)
    eligible = []                         # E(q), kept sorted
    for q in range(S):
        t = q - w
        if t >= s:
            bisect.insort(eligible, int(ranks[t]))
        if len(eligible) >= k:
            tau[q] = 0 if k == 0 else eligible[k - 1]
    return tau


def keep_mask(ranks: np.ndarray, s: int, w: int, k: int) -> np.ndarray:
    """[S, S] boolean: query q attends to key t (t <= q) if t is a sink
    (t < s), in the window (t > q - w), or eligible (s <= t <= q - w) with
    rank <= tau_q."""
    S = ranks.shape[0]
    tau = cutoffs(ranks, s, w, k)
    q = np.arange(S)[:, None]
    t = np.arange(S)[None, :]
    causal = t <= q
    sink = t < s
    window = t > q - w
    eligible = (t >= s) & (t <= q - w)
    return causal & (sink | window | (eligible & (ranks[None, :] <= tau[:, None])))
