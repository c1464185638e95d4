"""fp64 oracle: chunked prefill with a compression after every chunk.

TEST INFRASTRUCTURE ONLY (see the package docstring).

From the pages:

* KVP, section 4 ("Evaluation") and 4.1: long contexts are prefilled chunk
  by chunk and the cache is compressed after each chunk so that it stays
  within the budget; the retained rows are physically compacted. Budgets
  are uniform across heads.
* KVpop, "Delayed Memory Scoring": the normalisers are those of the sparse
  attention the model actually runs (over the keys it has retained), and
  the utility of the key at position t is the attention mass it receives
  from queries at positions d >= t + w.
* KVpop, "The KVpop Scoring Module" / Figure 1 and the pruning blog ("What
  we did"): the sink tokens and the most recent w tokens are always kept;
  the rest of the budget goes to the best-scored older tokens.

Readings where the pages leave the step open:

* The score of a cached key at a compression is the mass it receives from
  the queries of the chunk just appended (the only future queries that
  exist at that moment); each of those queries is normalised over the keys
  it can attend to, i.e. the retained earlier keys plus the chunk's own keys
  up to itself. Masses are summed over the query heads of a KV head.
* A budget is the total number of rows a head keeps, sinks and window
  included, the same for every head; with forced set F the head keeps
  min(n, max(budget, |F|)) rows. F is the sink positions 0 .. sinks-1 and
  the last `window` positions appended. Ties in mass go to the earlier
  position.

The cache of a KV head is a list of (position, k row, v row), kept in
position order. Everything here works on positions; nothing assumes that
row numbers and positions are related.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from .select_oracle import rank_candidates


def _default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def chunk_lse(q_chunk: np.ndarray, k_rows: np.ndarray, pos: np.ndarray, p0: int,
              scale: Optional[float] = None) -> np.ndarray:
    """Normalisers of a chunk's queries over the cached keys they can see.

    q_chunk ``[Hq, C, d]``: queries at positions p0 .. p0+C-1.
    k_rows ``[Hkv, n, d]`` and pos ``[Hkv, n]``: the cached keys (the chunk's
    own keys included) and their positions.
    ``lse[qh, i] = log sum_{r : pos[h, r] <= p0 + i} exp(scale <q, k_r>)``.
    """
    Hq, C, d = q_chunk.shape
    Hkv = k_rows.shape[0]
    g = Hq // Hkv
    scale = _default_scale(d) if scale is None else scale
    out = np.empty((Hq, C), dtype=np.float64)
    for qh in range(Hq):
        h = qh // g
        logit = (q_chunk[qh].astype(np.float64) @ k_rows[h].astype(np.float64).T) * scale
        visible = pos[h][None, :] <= (p0 + np.arange(C))[:, None]
        logit = np.where(visible, logit, -np.inf)
        top = logit.max(axis=1, keepdims=True)
        out[qh] = top[:, 0] + np.log(np.exp(logit - top).sum(axis=1))
    return out


def chunk_mass(q_chunk: np.ndarray, k_rows: np.ndarray, pos: np.ndarray, lse: np.ndarray,
               p0: int, W: int, scale: Optional[float] = None) -> np.ndarray:
    """Mass each cached key receives from the chunk's queries.

    ``mass[h, r] = sum_{qh in group h} sum_{i : p0 + i >= pos[h, r] + W}
    exp(scale <q_i, k_r> - lse[qh, i])`` (such a query sees the key, since
    W >= 0). Returns ``[Hkv, n]``.
    """
    Hq, C, d = q_chunk.shape
    Hkv, n = pos.shape
    g = Hq // Hkv
    scale = _default_scale(d) if scale is None else scale
    mass = np.zeros((Hkv, n), dtype=np.float64)
    for qh in range(Hq):
        h = qh // g
        logit = (q_chunk[qh].astype(np.float64) @ k_rows[h].astype(np.float64).T) * scale
        prob = np.exp(logit - lse[qh][:, None])
        counted = (p0 + np.arange(C))[:, None] >= pos[h][None, :] + W
        mass[h] += np.where(counted, prob, 0.0).sum(axis=0)
    return mass


class HeadCache:
    """One KV head's cache: positions and rows, in position order."""

    def __init__(self, d: int, dtype):
        self.pos = np.zeros(0, dtype=np.int64)
        self.k = np.zeros((0, d), dtype=dtype)
        self.v = np.zeros((0, d), dtype=dtype)

    def append(self, p0: int, k: np.ndarray, v: np.ndarray) -> None:
        self.pos = np.concatenate([self.pos, np.arange(p0, p0 + k.shape[0], dtype=np.int64)])
        self.k = np.concatenate([self.k, k])
        self.v = np.concatenate([self.v, v])

    def keep(self, rows: np.ndarray) -> None:
        rows = np.sort(np.asarray(rows, dtype=np.int64))
        self.pos, self.k, self.v = self.pos[rows], self.k[rows], self.v[rows]


def compress_rows(mass: np.ndarray, pos: np.ndarray, budget: int, sinks: int, window: int,
                  p_end: int) -> np.ndarray:
    """Rows (ascending) one head keeps: the forced positions (sinks, and the
    last `window` positions before p_end) and the best-scored others."""
    forced = (pos < sinks) | (pos >= p_end - window)
    n = pos.size
    keep_n = min(n, max(budget, int(forced.sum())))
    cand = np.flatnonzero(~forced)          # row order is position order
    chosen = rank_candidates(mass, cand)[:keep_n - int(forced.sum())]
    return np.sort(np.concatenate([np.flatnonzero(forced), chosen]))


def prefill_compress(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int, budget: int,
                     sinks: int, window: int, scale: Optional[float] = None,
                     record: Optional[List[dict]] = None) -> List[HeadCache]:
    """The chunked loop for one sequence: q ``[Hq, S, d]``, k, v ``[Hkv, S, d]``.

    For each chunk: append its keys, score every cached key with the chunk's
    queries (``chunk_lse``, ``chunk_mass``), and if a head holds more than
    the budget, keep ``compress_rows``. Returns the final per-head caches;
    ``record`` (if given) receives per chunk the positions scored, the lse,
    the mass and the rows kept.
    """
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    heads = [HeadCache(d, k.dtype) for _ in range(Hkv)]
    for p0 in range(0, S, chunk):
        p1 = min(S, p0 + chunk)
        for h in range(Hkv):
            heads[h].append(p0, k[h, p0:p1], v[h, p0:p1])
        pos = np.stack([hc.pos for hc in heads])
        krows = np.stack([hc.k for hc in heads])
        lse = chunk_lse(q[:, p0:p1], krows, pos, p0, scale)
        mass = chunk_mass(q[:, p0:p1], krows, pos, lse, p0, window, scale)
        kept = None
        if pos.shape[1] > budget:
            kept = [compress_rows(mass[h], pos[h], budget, sinks, window, p1) for h in range(Hkv)]
            for h in range(Hkv):
                heads[h].keep(kept[h])
        if record is not None:
            record.append({"p0": p0, "p1": p1, "pos": pos, "lse": lse, "mass": mass,
                           "kept_rows": kept})
    return heads
