"""KVpop supervision target from per-query-head future mass (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

KVpop, "Defining Future Attention Utility" (worked example) and the appendix
("Alternative Aggregation Methods"):

* count normalisation: key t can be seen by N_t = max(1, S - (t + w)) future
  queries (0-indexed positions t + w .. S - 1), and the mean future mass is
  the summed mass divided by N_t; this removes the advantage early tokens
  have from simply seeing more future queries;
* log transform: log(eps + mean mass);
* aggregation over the query heads g that share KV head h: the maximum of
  the logs, or alternatively the mean in probability space before the log.
"""
from __future__ import annotations

import numpy as np


def future_counts(S: int, w: int) -> np.ndarray:
    """``N_t = max(1, S - (t + w))`` for t = 0..S-1."""
    t = np.arange(S, dtype=np.int64)
    return np.maximum(1, S - (t + w)).astype(np.float64)


def target(per_query_head_mass: np.ndarray, w: int, eps: float = 0.0,
           aggregate: str = "max") -> np.ndarray:
    """Target ``[S]`` for one KV head from its group's masses ``[g, S]``.

    With ``eps = 0`` a key with no future query gets ``log 0 = -inf``.
    """
    m = np.asarray(per_query_head_mass, dtype=np.float64)
    g, S = m.shape
    mean = m / future_counts(S, w)[None, :]
    with np.errstate(divide="ignore"):
        if aggregate == "max":
            return np.log(eps + mean).max(axis=0)
        if aggregate == "mean":
            return np.log(eps + mean.mean(axis=0))
    raise ValueError(aggregate)
