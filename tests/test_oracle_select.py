"""Pins for the selection / compaction / budget oracle (CPU only).

Pins: pure-Python sorting with an explicit comparison key, exhaustive subset
enumeration for tiny n, the special cases named on the pages (sinks plus the
newest tokens; keep everything; keep only the forced set), the pages' budget
arithmetic, and the pruning blog's cache-size table.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import select_oracle as so
from future_attention_scoring_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_select(scores, budget, sinks, recent):
    """Pure Python: forced + best candidates by (non-NaN, score desc, pos asc)."""
    S = len(scores)
    forced = sorted(set(range(min(sinks, S))) | set(range(max(0, S - recent), S)))
    cand = [p for p in range(S) if p not in set(forced)]
    kept = min(S, max(budget, len(forced)))

    def key(p):
        s = scores[p]
        return (1 if math.isnan(s) else 0, 0.0 if math.isnan(s) else -s, p)

    chosen = sorted(cand, key=key)[: kept - len(forced)]
    return sorted(forced + chosen)


def beats(scores, a, b):
    """True if candidate a ranks above candidate b."""
    sa, sb = scores[a], scores[b]
    na, nb = math.isnan(sa), math.isnan(sb)
    if na != nb:
        return nb
    if not na and sa != sb:
        return sa > sb
    return a < b


def enumerate_select(scores, budget, sinks, recent):
    """Exhaustive: the unique k-subset whose members all beat all non-members."""
    S = len(scores)
    forced = sorted(set(range(min(sinks, S))) | set(range(max(0, S - recent), S)))
    cand = [p for p in range(S) if p not in set(forced)]
    n_choose = min(S, max(budget, len(forced))) - len(forced)
    winners = []
    for sub in itertools.combinations(cand, n_choose):
        rest = [p for p in cand if p not in sub]
        if all(beats(scores, a, b) for a in sub for b in rest):
            winners.append(sub)
    assert len(winners) == 1
    return sorted(forced + list(winners[0]))


def nasty_scores(rng, S):
    pool = np.array([0.0, -0.0, 1.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5, 1e-30, -1e-30, 3.0],
                    dtype=np.float32)
    s = rng.choice(pool, size=S).astype(np.float32)
    mix = rng.random(S) < 0.4
    s[mix] = rng.standard_normal(mix.sum()).astype(np.float32)
    return s


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_pure_python_sort(seed):
    rng = np.random.default_rng(seed)
    H, S = 3, int(rng.integers(1, 90))
    sinks, recent = int(rng.integers(0, 6)), int(rng.integers(0, 12))
    scores = np.stack([nasty_scores(rng, S) for _ in range(H)])
    budgets = [int(rng.integers(0, S + 5)) for _ in range(H)]
    idx, off = so.select(scores, budgets, sinks, recent)
    for h in range(H):
        assert idx[off[h]:off[h + 1]].tolist() == brute_select(scores[h].tolist(), budgets[h], sinks, recent)


@pytest.mark.parametrize("seed", range(8))
def test_select_matches_subset_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(4, 13))
    scores = nasty_scores(rng, S)
    sinks, recent = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    budget = int(rng.integers(0, S + 1))
    idx, _ = so.select(scores[None, :], [budget], sinks, recent)
    assert idx.tolist() == enumerate_select(scores.tolist(), budget, sinks, recent)


def test_sort_pin_rejects_reversed_tie_break():
    scores = np.zeros(20, dtype=np.float32)
    idx, _ = so.select(scores[None], [8], 2, 2)
    assert idx.tolist() == brute_select(scores.tolist(), 8, 2, 2)
    assert idx.tolist() == [0, 1, 2, 3, 4, 5, 18, 19]      # lower positions win ties


def test_scores_equal_to_position_give_sinks_plus_newest():
    # the blog's sinks-plus-recent policy: 4 sinks, the rest to the newest tokens
    S, b = 300, 64
    scores = np.arange(S, dtype=np.float32)
    idx, _ = so.select(scores[None], [b], 4, 32)
    assert idx.tolist() == list(range(4)) + list(range(S - (b - 4), S))


def test_budget_edges():
    S = 50
    scores = np.random.default_rng(0).standard_normal((1, S)).astype(np.float32)
    idx, off = so.select(scores, [S + 10], 4, 8)
    assert idx.tolist() == list(range(S))
    idx, off = so.select(scores, [3], 4, 8)
    assert idx.tolist() == list(range(4)) + list(range(42, 50))
    idx, off = so.select(scores, [0], 0, 0)
    assert idx.size == 0 and off.tolist() == [0, 0]
    # window covering everything
    idx, _ = so.select(scores, [5], 2, 100)
    assert idx.tolist() == list(range(S))


def test_plan_offsets():
    kept, off = so.plan([10, 2, 1000, 7], 100, 4, 4)
    assert kept.tolist() == [10, 8, 100, 8]
    assert off.tolist() == [0, 10, 18, 118, 126]


def test_budget_example_from_pages():
    with open(os.path.join(GOLDEN, "kvpop_budget_example.json")) as f:
        ex = json.load(f)
    n = ex["tokens"]
    forced = so.forced_positions(n, ex["sinks"], ex["window"])
    assert (forced + 1).tolist() == ex["forced_positions_1_indexed"]
    kept, _ = so.plan([ex["budget"]], n, ex["sinks"], ex["window"])
    assert kept[0] == ex["sinks"] + ex["window"] + ex["k"] == ex["budget"]
    scores = np.random.default_rng(1).random(n).astype(np.float32)
    idx, _ = so.select(scores[None], [ex["budget"]], ex["sinks"], ex["window"])
    assert idx.size == ex["budget"]
    assert set(forced.tolist()) <= set(idx.tolist())


def test_budgets_from_ratios_floor():
    assert so.budgets_from_ratios([0.15, 0.5, 0.999999], 1000).tolist() == [150, 500, 999]
    r = workloads.dirichlet_ratios(4, 8, 0.15)
    assert abs(r.mean() - 0.15) < 1e-12
    b = so.budgets_from_ratios(r, 131072)
    assert np.all(b == np.floor(r * 131072))


def test_compact_identity_and_gather():
    rng = np.random.default_rng(3)
    cache = rng.standard_normal((3, 40, 8)).astype(np.float16)
    idx = np.tile(np.arange(40, dtype=np.int32), 3)
    off = np.array([0, 40, 80, 120])
    out = so.compact(cache, idx, off)
    assert np.array_equal(out.view(np.int16), cache.reshape(120, 8).view(np.int16))
    idx2 = np.array([0, 5, 39, 1, 2, 7], dtype=np.int32)
    off2 = np.array([0, 3, 3, 6])
    out2 = so.compact(cache, idx2, off2)
    assert np.array_equal(out2[0], cache[0, 0]) and np.array_equal(out2[2], cache[0, 39])
    assert np.array_equal(out2[3], cache[2, 1]) and np.array_equal(out2[5], cache[2, 7])


def test_decode_sweep_cache_sizes_match_blog():
    with open(os.path.join(GOLDEN, "blog_cache_sizes.json")) as f:
        ex = json.load(f)
    cell = workloads.decode_sweep()[0]
    shape = ex["model_cache_shape"]
    assert (cell.layers, cell.kv_heads, cell.d) == (shape["layers"], shape["kv_heads"], shape["head_dim"])
    per_token = cell.H * cell.d * shape["tensors"] * np.dtype(np.float16).itemsize
    assert per_token == ex["kib_per_token"] * 1024
    for tokens, mib in ex["retained_tokens_to_mib"].items():
        assert int(tokens) * per_token == mib * 2 ** 20
    # the printed full-history figure is ~0.35 MiB above tokens * 28 KiB
    assert abs(120000 * per_token / 2 ** 20 - ex["full_history_120000_tokens_mib_printed"]) < 0.5
