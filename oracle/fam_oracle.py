"""fp64 oracle: causal row log-sum-exp and per-KV-head future-attention mass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, from the pages:

* KVpop, "Defining Future Attention Utility" and Figure 2 ("Transposed
  Attention"): the utility of key t is the attention mass it receives from
  queries d that come after it has left the protected window of w recent
  tokens, i.e. from queries with d >= t + w.
* KVpop, "Delayed Memory Scoring" (the LSE example): the normaliser of query
  d is LSE(d) = log of the sum of exp(logit) over the keys it may attend to,
  which under causal masking are the keys t' <= d (the query itself
  included).
* KVpop, "Delayed Memory Scoring" (the transposed pass) and the appendix
  section on obtaining targets by a transposed attention pass: subtract the
  original per-query normaliser from each logit and keep only d >= t + w.
* The softmax logit is <q, k> / sqrt(d) (KVpop, "Background: Linear
  Attention", where the printed kernel has the sqrt(d) misplaced; the
  standard reading is used).
* Aggregation over the query heads that share KV head h: a plain sum (the
  page takes a max of logs; the sum is the raw-mass reading used here).

Query head qh reads KV head qh // g with g = Hq // Hkv (contiguous groups).

Everything is dense fp64. Rows are processed in blocks only to bound memory:
every row's normaliser is formed from its complete row of logits, and every
mass is an explicit masked column sum of explicit softmax probabilities.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def _logits(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """fp64 logits ``scale * q_rows @ k.T``."""
    return (q_rows.astype(np.float64) @ k.astype(np.float64).T) * scale


def causal_lse_rows(q: np.ndarray, k: np.ndarray, rows: np.ndarray,
                    scale: float) -> np.ndarray:
    """LSE of the listed query rows of one head: ``log sum_{j<=i} exp(l_ij)``.

    q: ``[S, d]`` queries of one query head; k: ``[S, d]`` keys of its KV head.
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    for n, i in enumerate(rows):
        logit = _logits(q[i:i + 1], k[: i + 1], scale)[0]
        top = logit.max()
        out[n] = top + math.log(np.exp(logit - top).sum())
    return out


def causal_lse(q: np.ndarray, k: np.ndarray, scale: Optional[float] = None,
               block: int = 256) -> np.ndarray:
    """Per-query causal LSE for all heads.

    q: ``[Hq, S, d]``, k: ``[Hkv, S, d]`` -> ``[Hq, S]`` fp64 (natural log).
    """
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    g = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    lse = np.empty((Hq, S), dtype=np.float64)
    for qh in range(Hq):
        kh = k[qh // g]
        for r0 in range(0, S, block):
            r1 = min(S, r0 + block)
            logit = _logits(q[qh, r0:r1], kh[:r1], scale)
            i = np.arange(r0, r1)[:, None]
            j = np.arange(r1)[None, :]
            logit[j > i] = -np.inf                      # causal: keys j <= i
            top = logit.max(axis=1, keepdims=True)
            lse[qh, r0:r1] = top[:, 0] + np.log(np.exp(logit - top).sum(axis=1))
    return lse


def future_mass(q: np.ndarray, k: np.ndarray, lse: np.ndarray, W: int,
                scale: Optional[float] = None, block: int = 256,
                per_query_head: bool = False):
    """Future-attention mass per KV head.

    ``mass[h, j] = sum_{qh in group(h)} sum_{i >= j + W} exp(l_ij - lse[qh, i])``
    where ``l_ij`` is the causal logit (i >= j + W >= j, so every counted
    pair is causal). Keys with ``j > S - 1 - W`` receive exactly 0.

    Returns ``mass [Hkv, S]`` and, if ``per_query_head``, also ``[Hq, S]``.
    """
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    g = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    per_q = np.zeros((Hq, S), dtype=np.float64)
    for qh in range(Hq):
        kh = k[qh // g]
        for r0 in range(0, S, block):
            r1 = min(S, r0 + block)
            logit = _logits(q[qh, r0:r1], kh[:r1], scale)
            prob = np.exp(logit - lse[qh, r0:r1, None])
            i = np.arange(r0, r1)[:, None]
            j = np.arange(r1)[None, :]
            prob[i < j + W] = 0.0                        # only d >= t + w counts
            per_q[qh, :r1] += prob.sum(axis=0)
    mass = per_q.reshape(Hkv, g, S).sum(axis=1)
    if per_query_head:
        return mass, per_q
    return mass


def fam(q: np.ndarray, k: np.ndarray, W: int, scale: Optional[float] = None,
        block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Both outputs for ``q [B,Hq,S,d]`` / ``k [B,Hkv,S,d]`` (or without B)."""
    if q.ndim == 3:
        lse = causal_lse(q, k, scale, block)
        return lse, future_mass(q, k, lse, W, scale, block)
    lses, masses = [], []
    for b in range(q.shape[0]):
        lse = causal_lse(q[b], k[b], scale, block)
        lses.append(lse)
        masses.append(future_mass(q[b], k[b], lse, W, scale, block))
    return np.stack(lses), np.stack(masses)


def future_mass_keys(q_group: np.ndarray, k: np.ndarray, lse_tail: np.ndarray,
                     tail_start: int, keys: np.ndarray, W: int,
                     scale: Optional[float] = None) -> np.ndarray:
    """Mass of selected keys whose future queries all lie in a known tail.

    q_group: ``[g, S, d]`` the group's queries; lse_tail: ``[g, S - tail_start]``
    normalisers of rows ``tail_start..S-1``. Every key j must satisfy
    ``j + W >= tail_start`` so that all its counted queries are in the tail.
    """
    g, S, d = q_group.shape
    scale = default_scale(d) if scale is None else scale
    keys = np.asarray(keys, dtype=np.int64)
    if keys.size and keys.min() + W < tail_start:
        raise ValueError("a key's future queries start before the tail")
    out = np.zeros(keys.shape[0], dtype=np.float64)
    for n, j in enumerate(keys):
        i0 = j + W
        if i0 >= S:
            continue
        for qh in range(g):
            logit = _logits(q_group[qh, i0:], k[j:j + 1], scale)[:, 0]
            out[n] += np.exp(logit - lse_tail[qh, i0 - tail_start:]).sum()
    return out
