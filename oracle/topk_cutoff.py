"""Running top-k cut-off over static ranks (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages (KVpop, "Delayed Memory Scoring" and "Efficient Online
Pruning"): tokens are pre-sorted by a static priority score and ranked (rank
1 is the best); at query q the token t = q - w leaves the protected window
and becomes eligible; the cut-off tau_q is the rank of the k-th best
eligible token, and the attention keeps the sinks, the window and the
eligible tokens with rank <= tau_q. The page maintains the eligible ranks in
a Fenwick tree and finds tau_q by binary lifting; the value itself is an
order statistic, so the oracle computes it from that definition.

Readings where the pages are silent: ranks order the static scores
descending with ties to the lower position (as selection does); every token
that leaves the window becomes eligible, sinks included; with fewer than k
eligible tokens (or none) tau_q = S, so every eligible token passes
"rank <= tau_q"; with k = 0, tau_q = 0.
"""
from __future__ import annotations

import numpy as np

from .select_oracle import rank_candidates


def ranks_from_scores(scores: np.ndarray) -> np.ndarray:
    """Rank (1 = best) of every position of one head."""
    n = scores.shape[0]
    order = rank_candidates(scores, np.arange(n))
    ranks = np.empty(n, dtype=np.int64)
    ranks[order] = np.arange(1, n + 1)
    return ranks


def cutoffs(ranks: np.ndarray, w: int, k: int) -> np.ndarray:
    """tau_q for q = 0 .. S-1 of one head: the k-th smallest rank among the
    tokens t <= q - w, or S if fewer than k are eligible (0 if k = 0)."""
    S = ranks.shape[0]
    out = np.empty(S, dtype=np.int64)
    for q in range(S):
        if k == 0:
            out[q] = 0
            continue
        eligible = ranks[: max(0, q - w + 1)]
        out[q] = np.sort(eligible)[k - 1] if eligible.size >= k else S
    return out


def keep_mask(ranks: np.ndarray, w: int, k: int, sinks: int) -> np.ndarray:
    """[S, S] boolean: query q attends to key t (t <= q) if t is a sink, in
    the window (t > q - w), or eligible with rank <= tau_q."""
    S = ranks.shape[0]
    tau = cutoffs(ranks, w, k)
    q = np.arange(S)[:, None]
    t = np.arange(S)[None, :]
    causal = t <= q
    window = t > q - w
    eligible = t <= q - w
    return causal & ((t < sinks) | window | (eligible & (ranks[None, :] <= tau[:, None])))
