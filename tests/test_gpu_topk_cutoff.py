"""GPU parity of fam_topk_cutoff (KVpop's running top-k cut-off) against
oracle/topk_cutoff.py: integer results, compared exactly.

Ranks come from fam_rank_order on scores with ties; the oracle ranks the
same scores itself. Cases: the page's Fenwick-tree example, random shapes
(S not a multiple of the 2048-query chunk), k = 0, k > S, w >= S, S = 1,
several heads, and at 131072 positions the closed forms (older or newer
tokens ranked best) plus sampled queries of a random ranking; at the
largest S (262144: 256 tiles of 1024 positions, the most tile counts a
level sums), with many heads, on tile boundaries, and twice on one
workspace.
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


def gpu_cutoffs(scores: np.ndarray, w: int, k: int) -> np.ndarray:
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).to(DEV)
    return fam.fam_topk_cutoff(fam.fam_rank_order(s), w, k).cpu().numpy()


def test_page_example_on_gpu():
    with open(os.path.join(GOLDEN, "kvpop_fenwick_example.json")) as f:
        ex = json.load(f)
    say("fam_topk_cutoff on the page's Fenwick example")
    ranks = np.array(ex["inserted_ranks"] + [5, 2])
    scores = -ranks.astype(np.float32)              # rank 1 = highest score
    tau = gpu_cutoffs(scores[None], w=0, k=ex["k"])[0]
    assert tau[1] == ex["cutoff_after_second"] and tau[2] == ex["cutoff_after_third"]
    assert tau[0] == len(ranks)


@pytest.mark.parametrize("seed,H,S,w,k", [(0, 1, 1, 0, 1), (1, 3, 2500, 32, 100), (2, 2, 4097, 0, 1),
                                          (3, 4, 3000, 128, 2900), (4, 1, 2000, 2500, 5), (5, 2, 700, 7, 0),
                                          (6, 5, 6000, 64, 6001), (7, 8, 5000, 512, 1024)])
def test_cutoffs_match_oracle(seed, H, S, w, k):
    say(f"fam_topk_cutoff seed={seed} H={H} S={S} w={w} k={k}")
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((H, S)).astype(np.float32)
    scores[rng.random((H, S)) < 0.1] = 0.25
    got = gpu_cutoffs(scores, w, k)
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        np.testing.assert_array_equal(got[h], tc.cutoffs(ranks, w, k))


def test_closed_forms_at_131072():
    S, w, k, H = 131072, 512, 16384, 2
    say(f"fam_topk_cutoff closed forms S={S}")
    pos = np.arange(S, dtype=np.float32)
    got = gpu_cutoffs(np.stack([-pos, pos]), w, k)           # row 0: older better; row 1: newer better
    q = np.arange(S)
    want_old = np.where(q >= w + k - 1, k, S)
    want_new = np.where(q >= w + k - 1, S - (q - w) + k - 1, S)
    np.testing.assert_array_equal(got[0], want_old)
    np.testing.assert_array_equal(got[1], want_new)


def test_random_ranking_sampled_at_131072():
    S, w, k, H = 131072, 512, 8192, 4
    say(f"fam_topk_cutoff random scores S={S}, sampled queries")
    scores = np.random.default_rng(11).standard_normal((H, S)).astype(np.float32)
    got = gpu_cutoffs(scores, w, k)
    qs = np.array([0, w, w + k - 2, w + k - 1, w + k, 20000, 65536, 100001, S - 1])
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        for q in qs:
            elig = ranks[: max(0, q - w + 1)]
            want = np.partition(elig, k - 1)[k - 1] if elig.size >= k else S
            assert got[h, q] == want, (h, q)
        full = got[h, w + k - 1:]
        assert np.all(np.diff(full) <= 0)


@pytest.mark.parametrize("H,S", [(33, 3000), (3, 1024), (3, 1025), (2, 65536 + 7)])
def test_tile_boundaries_and_many_heads(H, S):
    say(f"fam_topk_cutoff H={H} S={S}")
    rng = np.random.default_rng(S + H)
    scores = rng.standard_normal((H, S)).astype(np.float32)
    w, k = 3, max(1, S // 7)
    got = gpu_cutoffs(scores, w, k)
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        np.testing.assert_array_equal(got[h], tc.cutoffs(ranks, w, k))


def test_largest_s_sampled_and_workspace_reuse():
    """S = 262144 on two heads, then a small call on the same workspace: each
    call clears its per-tile counts of ones."""
    S, w, k, H = 262144, 100, 50000, 2
    say(f"fam_topk_cutoff S={S} then S=3000 on one workspace")
    ws = torch.empty(fam.fam_topk_cutoff_workspace_size(H, S), dtype=torch.uint8, device=DEV)
    scores = np.random.default_rng(12).standard_normal((H, S)).astype(np.float32)
    order = fam.fam_rank_order(torch.from_numpy(scores).to(DEV))
    got = fam.fam_topk_cutoff(order, w, k, workspace=ws).cpu().numpy()
    qs = np.array([w + k - 2, w + k - 1, 70000, 131071, 131072, 200003, S - 1])
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        for q in qs:
            elig = ranks[: max(0, q - w + 1)]
            want = np.partition(elig, k - 1)[k - 1] if elig.size >= k else S
            assert got[h, q] == want, (h, q)
        assert np.all(np.diff(got[h, w + k - 1:]) <= 0)
    small = np.random.default_rng(13).standard_normal((3, 3000)).astype(np.float32)
    order = fam.fam_rank_order(torch.from_numpy(small).to(DEV))
    got = fam.fam_topk_cutoff(order, 5, 200, workspace=ws).cpu().numpy()
    for h in range(3):
        np.testing.assert_array_equal(got[h], tc.cutoffs(tc.ranks_from_scores(small[h].astype(np.float64)), 5, 200))
