"""Pins for the running top-k cut-off oracle (CPU only).

oracle/topk_cutoff.py is checked against:
  * the page's Fenwick-tree example (tests/golden/kvpop_fenwick_example.json):
    ranks 3, 1, 4 inserted with k = 2 give the cut-off 3, then still 3,
  * brute force in pure Python (sorted eligible ranks per query),
  * a Fenwick tree with binary lifting written out as the page describes
    (insert the newly eligible rank, find the k-th by prefix count),
  * closed forms: ranks by age (older better) give tau_q = k once k tokens
    are eligible; ranks by recency (newer better) give S - (q - w) + k - 1,
  * the special cases k = 0, k larger than every eligible set, w >= S,
and the keep mask's row sizes (sinks + window + min(k, eligible) when no
sink is eligible and ranked in the top k).
"""
import json
import os

import numpy as np
import pytest

from oracle import topk_cutoff as tc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def fenwick_cutoffs(ranks, w, k):
    """The page's procedure: a Fenwick tree over ranks 1..S, one insertion per
    query, the k-th rank found by binary lifting."""
    S = len(ranks)
    tree = [0] * (S + 1)
    top = 1 << (S.bit_length())
    out, n_elig = [], 0
    for q in range(S):
        t = q - w
        if t >= 0:
            i = int(ranks[t])
            while i <= S:
                tree[i] += 1
                i += i & -i
            n_elig += 1
        if k == 0:
            out.append(0)
        elif n_elig < k:
            out.append(S)
        else:
            pos, rem, step = 0, k, top
            while step:
                if pos + step <= S and tree[pos + step] < rem:
                    pos += step
                    rem -= tree[pos]
                step >>= 1
            out.append(pos + 1)
    return np.array(out)


def test_page_example():
    with open(os.path.join(GOLDEN, "kvpop_fenwick_example.json")) as f:
        ex = json.load(f)
    ranks = np.array(ex["inserted_ranks"] + [5, 2])      # tree of length 5: the other ranks arrive later
    tau = tc.cutoffs(ranks, w=0, k=ex["k"])
    assert tau[1] == ex["cutoff_after_second"] and tau[2] == ex["cutoff_after_third"]
    counts = np.bincount(ranks[:2], minlength=ex["tree_length"] + 1)[1:]
    assert counts.tolist() == ex["counts_after_first_two"]
    assert tau[0] == len(ranks)                           # one eligible token, fewer than k


@pytest.mark.parametrize("seed,S,w,k", [(0, 1, 0, 1), (1, 30, 3, 4), (2, 57, 0, 10), (3, 80, 7, 1),
                                        (4, 64, 10, 60), (5, 40, 45, 3)])
def test_against_brute_force_and_fenwick(seed, S, w, k):
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal(S)
    scores[rng.random(S) < 0.2] = 0.0                      # ties
    ranks = tc.ranks_from_scores(scores)
    assert sorted(ranks.tolist()) == list(range(1, S + 1))
    got = tc.cutoffs(ranks, w, k)
    brute = []
    for q in range(S):
        el = sorted(int(ranks[t]) for t in range(S) if t <= q - w)
        brute.append(el[k - 1] if len(el) >= k else S)
    assert got.tolist() == brute
    assert got.tolist() == fenwick_cutoffs(ranks, w, k).tolist()
    # once k tokens are eligible the cut-off never rises
    full = got[w + k - 1:] if w + k - 1 < S else got[:0]
    assert np.all(np.diff(full) <= 0)


def test_closed_forms_and_special_cases():
    S, w, k = 200, 16, 12
    older_better = np.arange(1, S + 1)
    tau = tc.cutoffs(older_better, w, k)
    assert np.all(tau[w + k - 1:] == k) and np.all(tau[:w + k - 1] == S)
    newer_better = S - np.arange(S)
    tau = tc.cutoffs(newer_better, w, k)
    q = np.arange(w + k - 1, S)
    assert np.array_equal(tau[w + k - 1:], S - (q - w) + k - 1)
    assert np.all(tc.cutoffs(older_better, w, 0) == 0)
    assert np.all(tc.cutoffs(older_better, S, k) == S)
    assert np.all(tc.cutoffs(older_better, 0, S + 5) == S)


def test_keep_mask_row_sizes():
    S, w, k, sinks = 120, 8, 10, 0
    ranks = tc.ranks_from_scores(np.random.default_rng(7).standard_normal(S))
    m = tc.keep_mask(ranks, w, k, sinks)
    for q in range(S):
        n_elig = max(0, q - w + 1)
        assert m[q].sum() == min(q + 1, w) + min(k, n_elig)
