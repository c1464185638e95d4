"""Pins for the running top-k cut-off oracle (CPU only).

oracle/topk_cutoff.py follows KVpop Algorithm 2 (budget (s, w, k); tau_q
starts at -1; the token t = q - w is inserted only if t >= s; tau_q is set
only once |E(q)| >= k). It is checked against:
  * Algorithm 2 transcribed as a Fenwick tree over ranks 1..S with the
    t >= s guard and a binary-lifting prefix-count search,
  * brute force in pure Python (the sorted eligible ranks of every query),
  * cut-offs worked out by hand from the page's six-token rank example
    (tests/golden/kvpop_rank_example.json) for s = 0 and s = 1,
  * the page's Fenwick-tree example (tests/golden/kvpop_fenwick_example.json):
    ranks 3, 1, 4 inserted with k = 2 give the cut-off 3, then still 3,
  * closed forms: ranks by age (older better) give tau_q = s + k once k
    tokens are eligible; ranks by recency (newer better) give
    S - (q - w) + k - 1,
  * the special cases k = 0, k larger than every eligible set, w >= S,
    s >= S,
and the direction of ranks_from_scores (rank 1 = highest score, ties to the
lower position) and the keep mask's row sizes with sinks.
"""
import json
import os

import numpy as np
import pytest

from oracle import topk_cutoff as tc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def algorithm2_fenwick(ranks, s, w, k):
    """Algorithm 2 step by step: a Fenwick tree T of counts over ranks
    1..S; FindByPrefixCount(T, k) is the smallest rank whose prefix count
    reaches k (0 when k = 0), found by binary lifting."""
    S = len(ranks)
    T = [0] * (S + 1)

    def insert(r):
        while r <= S:
            T[r] += 1
            r += r & -r

    def find_by_prefix_count(kk):
        if kk == 0:
            return 0
        pos, rem, step = 0, kk, 1 << S.bit_length()
        while step:
            if pos + step <= S and T[pos + step] < rem:
                pos += step
                rem -= T[pos]
            step >>= 1
        return pos + 1

    tau = [-1] * S
    n_eligible = 0
    for q in range(S):
        t = q - w
        if t >= s:
            insert(int(ranks[t]))
            n_eligible += 1
        if n_eligible >= k:
            tau[q] = find_by_prefix_count(k)
    return np.array(tau)


def brute(ranks, s, w, k):
    S = len(ranks)
    out = []
    for q in range(S):
        el = sorted(int(ranks[t]) for t in range(S) if s <= t <= q - w)
        out.append(-1 if len(el) < k else (0 if k == 0 else el[k - 1]))
    return np.array(out)


def test_page_rank_example_by_hand():
    """The page's ranks (token 0..5 have ranks 2, 6, 3, 1, 5, 4), w = 2, k = 2.
    s = 0: q = 2 inserts token 0 (rank 2), one eligible -> -1; q = 3 inserts
    rank 6 -> {2, 6} -> 6; q = 4 inserts rank 3 -> {2, 3, 6} -> 3; q = 5
    inserts rank 1 -> {1, 2, 3, 6} -> 2.
    s = 1: token 0 is a sink and never inserted; q = 3 inserts rank 6, one
    eligible -> -1; q = 4 inserts rank 3 -> {3, 6} -> 6; q = 5 inserts rank 1
    -> {1, 3, 6} -> 3."""
    with open(os.path.join(GOLDEN, "kvpop_rank_example.json")) as f:
        ranks = np.array(json.load(f)["rank_of_token"])
    assert tc.cutoffs(ranks, 0, 2, 2).tolist() == [-1, -1, -1, 6, 3, 2]
    assert tc.cutoffs(ranks, 1, 2, 2).tolist() == [-1, -1, -1, -1, 6, 3]
    assert tc.cutoffs(ranks, 2, 2, 1).tolist() == [-1, -1, -1, -1, 3, 1]


def test_page_fenwick_example():
    with open(os.path.join(GOLDEN, "kvpop_fenwick_example.json")) as f:
        ex = json.load(f)
    ranks = np.array(ex["inserted_ranks"] + [5, 2])      # tree of length 5: the other ranks arrive later
    tau = tc.cutoffs(ranks, 0, 0, ex["k"])
    assert tau[1] == ex["cutoff_after_second"] and tau[2] == ex["cutoff_after_third"]
    counts = np.bincount(ranks[:2], minlength=ex["tree_length"] + 1)[1:]
    assert counts.tolist() == ex["counts_after_first_two"]
    assert tau[0] == -1                                   # one eligible token, fewer than k


@pytest.mark.parametrize("seed,S,s,w,k", [(0, 1, 0, 0, 1), (1, 30, 0, 3, 4), (2, 57, 4, 0, 10),
                                          (3, 80, 1, 7, 1), (4, 64, 4, 10, 50), (5, 40, 0, 45, 3),
                                          (6, 90, 12, 5, 0), (7, 70, 3, 2, 66), (8, 50, 60, 1, 1)])
def test_against_brute_force_and_fenwick(seed, S, s, w, k):
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal(S)
    scores[rng.random(S) < 0.2] = 0.0                      # ties
    ranks = tc.ranks_from_scores(scores)
    assert sorted(ranks.tolist()) == list(range(1, S + 1))
    got = tc.cutoffs(ranks, s, w, k)
    assert got.tolist() == brute(ranks, s, w, k).tolist()
    assert got.tolist() == algorithm2_fenwick(ranks, s, w, k).tolist()
    # once k tokens are eligible the cut-off never rises; before, it is -1
    if k == 0:
        assert np.all(got == 0)
        return
    first = s + w + k - 1
    assert np.all(got[:min(first, S)] == -1)
    if first < S:
        assert np.all(got[first:] >= 0) and np.all(np.diff(got[first:]) <= 0)


def test_closed_forms_and_special_cases():
    S, w, k = 200, 16, 12
    for s in (0, 1, 4):
        first = s + w + k - 1
        older_better = np.arange(1, S + 1)
        tau = tc.cutoffs(older_better, s, w, k)
        assert np.all(tau[first:] == s + k) and np.all(tau[:first] == -1)
        newer_better = S - np.arange(S)
        tau = tc.cutoffs(newer_better, s, w, k)
        q = np.arange(first, S)
        assert np.array_equal(tau[first:], S - (q - w) + k - 1) and np.all(tau[:first] == -1)
    older_better = np.arange(1, S + 1)
    assert np.all(tc.cutoffs(older_better, 4, w, 0) == 0)
    assert np.all(tc.cutoffs(older_better, 4, S, k) == -1)
    assert np.all(tc.cutoffs(older_better, S, 0, 1) == -1)
    assert np.all(tc.cutoffs(older_better, 0, 0, S + 5) == -1)
    assert tc.cutoffs(older_better, 0, 0, S)[-1] == S


def test_rank_direction():
    """Rank 1 is the highest score; ties go to the lower position; NaN last.
    The scores below rank exactly as the page's Fenwick-tree example."""
    assert tc.ranks_from_scores(np.arange(6, dtype=np.float64)).tolist() == [6, 5, 4, 3, 2, 1]
    assert tc.ranks_from_scores(np.zeros(4)).tolist() == [1, 2, 3, 4]
    assert tc.ranks_from_scores(np.array([0.5, 2.0, 0.5, -1.0, 2.0])).tolist() == [3, 1, 4, 5, 2]
    assert tc.ranks_from_scores(np.array([np.nan, -np.inf, 1.0, np.nan])).tolist() == [3, 2, 1, 4]


@pytest.mark.parametrize("s,w,k", [(0, 8, 10), (4, 8, 10), (4, 1, 3), (9, 20, 30)])
def test_keep_mask_row_sizes(s, w, k):
    S = 120
    ranks = tc.ranks_from_scores(np.random.default_rng(7).standard_normal(S))
    m = tc.keep_mask(ranks, s, w, k)
    tau = tc.cutoffs(ranks, s, w, k)
    for q in range(S):
        forced = sum(1 for t in range(q + 1) if t < s or t > q - w)
        n_elig = sum(1 for t in range(q + 1) if s <= t <= q - w)
        assert m[q].sum() == forced + (k if n_elig >= k else 0)
        kept_elig = [t for t in range(q + 1) if s <= t <= q - w and m[q, t]]
        if n_elig >= k:
            assert max((ranks[t] for t in kept_elig), default=0) == max(tau[q], 0)
        assert all(m[q, t] for t in range(min(s, q + 1)))   # every causal sink is kept
