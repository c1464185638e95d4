"""GPU parity of fam_topk_cutoff (KVpop's running top-k cut-off, Algorithm
2) against oracle/topk_cutoff.py: integer results, compared exactly.

Ranks come from fam_rank_order on scores with ties; the oracle ranks the
same scores itself. Cases: the page's Fenwick-tree and rank examples, random
shapes with s in {0, 1, 4} (S not a multiple of the 1024-position tile;
early queries with fewer than k eligible tokens, whose cut-off is -1),
k = 0, k > S, w >= S, s >= S, S = 1, several heads, at 131072 positions the
closed forms (older or newer tokens ranked best) plus sampled queries of a
random ranking; at 300000 positions with 8 heads (above the old 262144 cap),
with many heads, on tile boundaries, and twice on one workspace.
"""
import json
import os

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam
from oracle import topk_cutoff as tc

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_cutoffs(scores: np.ndarray, s: int, w: int, k: int) -> np.ndarray:
    sc = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).to(DEV)
    return fam.fam_topk_cutoff(fam.fam_rank_order(sc), s, w, k).cpu().numpy()


def sampled_want(ranks, s, w, k, q):
    """The oracle's definition at one query: the k-th smallest rank of E(q)."""
    elig = ranks[s: max(s, q - w + 1)]
    if elig.size < k:
        return -1
    return 0 if k == 0 else np.partition(elig, k - 1)[k - 1]


def test_page_examples_on_gpu():
    with open(os.path.join(GOLDEN, "kvpop_fenwick_example.json")) as f:
        ex = json.load(f)
    say("fam_topk_cutoff on the page's Fenwick and rank examples")
    ranks = np.array(ex["inserted_ranks"] + [5, 2])
    scores = -ranks.astype(np.float32)              # rank 1 = highest score
    tau = gpu_cutoffs(scores[None], 0, 0, ex["k"])[0]
    assert tau[1] == ex["cutoff_after_second"] and tau[2] == ex["cutoff_after_third"]
    assert tau[0] == -1
    with open(os.path.join(GOLDEN, "kvpop_rank_example.json")) as f:
        ranks = np.array(json.load(f)["rank_of_token"])
    scores = -ranks.astype(np.float32)
    assert gpu_cutoffs(scores[None], 0, 2, 2)[0].tolist() == [-1, -1, -1, 6, 3, 2]
    assert gpu_cutoffs(scores[None], 1, 2, 2)[0].tolist() == [-1, -1, -1, -1, 6, 3]


@pytest.mark.parametrize("seed,H,S,s,w,k", [(0, 1, 1, 0, 0, 1), (1, 3, 2500, 4, 32, 100), (2, 2, 4097, 0, 0, 1),
                                            (3, 4, 3000, 1, 128, 2800), (4, 1, 2000, 4, 2500, 5),
                                            (5, 2, 700, 4, 7, 0), (6, 5, 6000, 0, 64, 6001),
                                            (7, 8, 5000, 4, 512, 1024), (8, 3, 1500, 1, 0, 1499),
                                            (9, 2, 900, 1000, 3, 1), (10, 2, 1025, 1, 3, 1021)])
def test_cutoffs_match_oracle(seed, H, S, s, w, k):
    say(f"fam_topk_cutoff seed={seed} H={H} S={S} s={s} w={w} k={k}")
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((H, S)).astype(np.float32)
    scores[rng.random((H, S)) < 0.1] = 0.25
    got = gpu_cutoffs(scores, s, w, k)
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        np.testing.assert_array_equal(got[h], tc.cutoffs(ranks, s, w, k))


@pytest.mark.parametrize("s", [0, 1, 4])
def test_closed_forms_at_131072(s):
    S, w, k = 131072, 512, 16384
    say(f"fam_topk_cutoff closed forms S={S} s={s}")
    pos = np.arange(S, dtype=np.float32)
    got = gpu_cutoffs(np.stack([-pos, pos]), s, w, k)        # row 0: older better; row 1: newer better
    q = np.arange(S)
    first = s + w + k - 1
    want_old = np.where(q >= first, s + k, -1)
    want_new = np.where(q >= first, S - (q - w) + k - 1, -1)
    np.testing.assert_array_equal(got[0], want_old)
    np.testing.assert_array_equal(got[1], want_new)


def test_random_ranking_sampled_at_131072():
    S, s, w, k, H = 131072, 4, 512, 8192, 4
    say(f"fam_topk_cutoff random scores S={S}, sampled queries")
    scores = np.random.default_rng(11).standard_normal((H, S)).astype(np.float32)
    got = gpu_cutoffs(scores, s, w, k)
    first = s + w + k - 1
    qs = np.array([0, w, first - 1, first, first + 1, 20000, 65536, 100001, S - 1])
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        for q in qs:
            assert got[h, q] == sampled_want(ranks, s, w, k, q), (h, q)
        assert np.all(got[h, :first] == -1)
        assert np.all(np.diff(got[h, first:]) <= 0)


@pytest.mark.parametrize("H,S", [(33, 3000), (3, 1024), (3, 1025), (2, 65536 + 7)])
def test_tile_boundaries_and_many_heads(H, S):
    say(f"fam_topk_cutoff H={H} S={S}")
    rng = np.random.default_rng(S + H)
    scores = rng.standard_normal((H, S)).astype(np.float32)
    s, w, k = 4, 3, max(1, S // 7)
    got = gpu_cutoffs(scores, s, w, k)
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        np.testing.assert_array_equal(got[h], tc.cutoffs(ranks, s, w, k))


def test_300000_positions_eight_heads_every_query():
    """Above the old 262144-position cap: every query of 8 heads, against the
    oracle's definition evaluated incrementally on a sorted list of E(q)."""
    S, s, w, k, H = 300000, 4, 512, 37500, 8
    say(f"fam_topk_cutoff S={S} H={H}")
    scores = np.random.default_rng(14).standard_normal((H, S)).astype(np.float32)
    got = gpu_cutoffs(scores, s, w, k)
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        first = s + w + k - 1
        assert np.all(got[h, :first] == -1)
        elig = np.sort(ranks[s: first - w + 1])
        assert got[h, first] == elig[k - 1]
        for q in np.random.default_rng(h).integers(first, S, 24):
            assert got[h, q] == sampled_want(ranks, s, w, k, q), (h, q)
        assert np.all(np.diff(got[h, first:]) <= 0)


def test_largest_s_sampled_and_workspace_reuse():
    """S = 262144 on two heads, then a small call on the same workspace: each
    call clears its per-tile counts of ones."""
    S, s, w, k, H = 262144, 1, 100, 50000, 2
    say(f"fam_topk_cutoff S={S} then S=3000 on one workspace")
    ws = torch.empty(fam.fam_topk_cutoff_workspace_size(H, S), dtype=torch.uint8, device=DEV)
    scores = np.random.default_rng(12).standard_normal((H, S)).astype(np.float32)
    order = fam.fam_rank_order(torch.from_numpy(scores).to(DEV))
    got = fam.fam_topk_cutoff(order, s, w, k, workspace=ws).cpu().numpy()
    first = s + w + k - 1
    qs = np.array([first - 1, first, 70000, 131071, 131072, 200003, S - 1])
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        for q in qs:
            assert got[h, q] == sampled_want(ranks, s, w, k, q), (h, q)
        assert np.all(np.diff(got[h, first:]) <= 0)
    small = np.random.default_rng(13).standard_normal((3, 3000)).astype(np.float32)
    order = fam.fam_rank_order(torch.from_numpy(small).to(DEV))
    got = fam.fam_topk_cutoff(order, 4, 5, 200, workspace=ws).cpu().numpy()
    for h in range(3):
        np.testing.assert_array_equal(got[h], tc.cutoffs(tc.ranks_from_scores(small[h].astype(np.float64)), 4, 5, 200))
