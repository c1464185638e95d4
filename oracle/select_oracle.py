"""Budget plan, sort-based top-k selection and compaction (fp64 / numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages:

* KVpop, "The KVpop Scoring Module" and Figure 1: the cache always keeps the
  sink tokens and a protected recent window; the rest of the per-head budget
  B = sinks + window + k goes to the top-k scored long-range tokens (the
  page's example keeps 2 sinks + 3 recent + 4 chosen = 9).
* KVP (Learning to Evict from Key-Value Cache), section 3: a ranking's top-b
  entries form the cache; eviction drops the lowest-ranked entries to meet a
  budget. Appendix A.2: the first 4 and the last 16 tokens are always kept.
* LKV, "LKV-H: Learning Global Budget Allocation": the per-head budget is
  b = floor(r * t) for a frozen ratio r and current length t.
* The pruning blog, "What we did": keep the first four tokens, the newest 32,
  and fill the remaining space with the highest-scoring older tokens.
* KVP, section 4.1 / A.2 and the blog's systems test: retained rows are
  physically copied into a new, smaller tensor.

Readings where the pages are silent: budgets are totals that include the
forced tokens; a budget below the forced count keeps the forced set only; a
budget above S keeps everything; ties in score go to the lower position;
-0.0 equals +0.0; NaN ranks below every number (and NaNs tie by position);
kept positions are emitted in ascending order; heads are packed one after
another (ragged rows with int64 offsets).
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def forced_positions(S: int, sinks: int, recent: int) -> np.ndarray:
    """Sorted positions kept regardless of score: ``[0,sinks) U [S-recent,S)``."""
    f = set(range(min(sinks, S))) | set(range(max(0, S - recent), S))
    return np.array(sorted(f), dtype=np.int64)


def candidate_positions(S: int, sinks: int, recent: int) -> np.ndarray:
    """Positions that compete on score: not a sink and not in the window."""
    forced = set(forced_positions(S, sinks, recent).tolist())
    return np.array([p for p in range(S) if p not in forced], dtype=np.int64)


def plan(budgets: Sequence[int], S: int, sinks: int, recent: int
         ) -> Tuple[np.ndarray, np.ndarray]:
    """Rows kept per head and packed offsets ``[H+1]``."""
    n_forced = forced_positions(S, sinks, recent).size
    kept = np.array([min(S, max(int(b), n_forced)) for b in budgets], dtype=np.int64)
    offsets = np.zeros(len(kept) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    return kept, offsets


def budgets_from_ratios(ratios: Sequence[float], t: int) -> np.ndarray:
    """``b_h = floor(r_h * t)`` in fp64."""
    return np.array([math.floor(float(r) * t) for r in ratios], dtype=np.int64)


def rank_candidates(scores: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """Candidates ordered best first: score descending, position ascending.

    NaN is worse than any number; -0.0 is canonicalised to +0.0 so that it
    ties with +0.0.
    """
    s = scores[cand].astype(np.float64) + 0.0          # -0.0 + 0.0 == +0.0
    nan = np.isnan(s)
    s = np.where(nan, 0.0, s)
    # lexsort: last key is primary. Non-NaN first, then higher score, then
    # lower position.
    order = np.lexsort((cand, -s, nan.astype(np.int8)))
    return cand[order]


def select(scores: np.ndarray, budgets: Sequence[int], sinks: int, recent: int
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Per-head kept positions, ascending, packed: ``idx [sum kept]`` int32."""
    H, S = scores.shape
    kept, offsets = plan(budgets, S, sinks, recent)
    forced = forced_positions(S, sinks, recent)
    cand = candidate_positions(S, sinks, recent)
    idx = np.empty(int(offsets[-1]), dtype=np.int32)
    for h in range(H):
        n_choose = int(kept[h]) - forced.size
        chosen = rank_candidates(scores[h], cand)[:n_choose]
        idx[offsets[h]:offsets[h + 1]] = np.sort(np.concatenate([forced, chosen]))
    return idx, offsets


def compact(cache: np.ndarray, idx: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Copy the kept rows of ``cache [H, S, d]`` into ``[sum kept, d]``."""
    H = cache.shape[0]
    parts = [cache[h][idx[offsets[h]:offsets[h + 1]].astype(np.int64)] for h in range(H)]
    if not parts:
        return cache.reshape(0, cache.shape[-1])[:0]
    return np.concatenate(parts, axis=0)
