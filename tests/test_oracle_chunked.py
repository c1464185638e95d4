"""Pins for the chunked prefill-compress oracle (CPU only).

oracle/chunked.py is checked against things other than itself:
  * brute force as pure-Python loops with math.fsum, on caches whose
    positions have gaps (as after evictions),
  * the no-eviction reduction: with a budget of at least S every chunk's
    normalisers are the dense causal ones, and the chunks' masses add up,
    key by key, to the dense future mass of the whole sequence,
  * the W = 0 invariant (every query's probabilities over its visible keys
    sum to one, so a KV head's masses from one chunk sum to g * C),
  * the uniform-logit closed form of the kept set: with q = 0 every key
    that all of a chunk's queries count gets the same, largest mass, so ties
    keep the earliest positions and the final cache holds exactly
    [0, budget - W) and the last W positions,
  * a brute-force loop (explicit lists, sorted by (-mass, position)),
  * the cache invariants after every compression,
and each pin is shown to reject a plausible mistake.
"""
import math

import numpy as np
import pytest

from oracle import chunked as ch
from oracle import fam_oracle as fo


def rand(seed, Hq, Hkv, S, d, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, S, d)) * spread
    k = rng.standard_normal((Hkv, S, d)) * spread
    v = rng.standard_normal((Hkv, S, d))
    return q, k, v


def brute_chunk(q_chunk, k_rows, pos, p0, W, scale):
    Hq, C, d = q_chunk.shape
    Hkv, n = pos.shape
    g = Hq // Hkv
    lse = np.zeros((Hq, C))
    logit = {}
    for qh in range(Hq):
        h = qh // g
        for i in range(C):
            vis = [r for r in range(n) if pos[h][r] <= p0 + i]
            xs = []
            for r in vis:
                x = math.fsum(q_chunk[qh][i][c] * k_rows[h][r][c] for c in range(d)) * scale
                logit[qh, i, r] = x
                xs.append(x)
            top = max(xs)
            lse[qh, i] = top + math.log(math.fsum(math.exp(x - top) for x in xs))
    mass = np.zeros((Hkv, n))
    for h in range(Hkv):
        for r in range(n):
            terms = [math.exp(logit[qh, i, r] - lse[qh, i])
                     for qh in range(h * g, (h + 1) * g) for i in range(C)
                     if p0 + i >= pos[h][r] + W]
            mass[h, r] = math.fsum(terms)
    return lse, mass


@pytest.mark.parametrize("seed,Hq,Hkv,d,W", [(0, 2, 1, 4, 0), (1, 4, 2, 4, 2), (2, 2, 2, 8, 5),
                                              (3, 3, 1, 4, 40)])
def test_chunk_scores_match_brute_force_with_gaps(seed, Hq, Hkv, d, W):
    rng = np.random.default_rng(100 + seed)
    p0, C = 20, 6
    old = [np.sort(rng.choice(p0, size=9, replace=False)) for _ in range(Hkv)]
    pos = np.stack([np.concatenate([o, np.arange(p0, p0 + C)]) for o in old])
    k_rows = rng.standard_normal((Hkv, pos.shape[1], d))
    q_chunk = rng.standard_normal((Hq, C, d))
    scale = 1 / math.sqrt(d)
    lse = ch.chunk_lse(q_chunk, k_rows, pos, p0, scale)
    mass = ch.chunk_mass(q_chunk, k_rows, pos, lse, p0, W, scale)
    lse_b, mass_b = brute_chunk(q_chunk, k_rows, pos, p0, W, scale)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mass, mass_b, rtol=1e-12, atol=1e-15)
    # a window taken strictly (d > t + w) would differ wherever a key sits
    # exactly W positions before a chunk query
    strict = ch.chunk_mass(q_chunk, k_rows, pos, lse, p0, W + 1, scale)
    hit = (pos + W >= p0) & (pos + W < p0 + C)
    if hit.any():
        assert not np.allclose(strict[hit], mass_b[hit], rtol=1e-9)


@pytest.mark.parametrize("W", [0, 3, 11])
def test_no_eviction_reduces_to_the_dense_oracle(W):
    Hq, Hkv, S, d, C = 4, 2, 45, 8, 10
    q, k, v = rand(7, Hq, Hkv, S, d)
    rec = []
    heads = ch.prefill_compress(q, k, v, C, budget=S, sinks=2, window=W, record=rec)
    lse_d = fo.causal_lse(q, k)
    mass_d = fo.future_mass(q, k, lse_d, W)
    total = np.zeros((Hkv, S))
    for r in rec:
        np.testing.assert_array_equal(r["pos"], np.tile(np.arange(r["p1"]), (Hkv, 1)))
        np.testing.assert_allclose(r["lse"], lse_d[:, r["p0"]:r["p1"]], rtol=0, atol=1e-12)
        total[:, :r["p1"]] += r["mass"]
        assert r["kept_rows"] is None
    np.testing.assert_allclose(total, mass_d, rtol=1e-11, atol=1e-14)
    for h in range(Hkv):
        np.testing.assert_array_equal(heads[h].pos, np.arange(S))
        np.testing.assert_array_equal(heads[h].k, k[h])


def test_w0_masses_of_a_chunk_sum_to_g_times_c():
    Hq, Hkv, S, d, C = 6, 2, 60, 8, 16
    q, k, v = rand(8, Hq, Hkv, S, d, spread=1.5)
    rec = []
    ch.prefill_compress(q, k, v, C, budget=20, sinks=3, window=0, record=rec)
    for r in rec:
        n_q = r["p1"] - r["p0"]
        np.testing.assert_allclose(r["mass"].sum(axis=1), (Hq // Hkv) * n_q, rtol=1e-12)


@pytest.mark.parametrize("S,C,budget,sinks,W", [(100, 16, 30, 4, 8), (97, 20, 25, 2, 5),
                                                 (64, 7, 16, 4, 3), (80, 10, 12, 4, 8)])
def test_uniform_logits_keep_the_earliest_and_the_window(S, C, budget, sinks, W):
    Hq, Hkv, d = 2, 2, 4
    _, k, v = rand(9, Hq, Hkv, S, d)
    q = np.zeros((Hq, S, d))
    heads = ch.prefill_compress(q, k, v, C, budget, sinks, W)
    keep = max(budget, sinks + W)
    want = np.concatenate([np.arange(keep - W), np.arange(S - W, S)])
    for h in range(Hkv):
        np.testing.assert_array_equal(heads[h].pos, want)
        np.testing.assert_array_equal(heads[h].k, k[h][want])
        np.testing.assert_array_equal(heads[h].v, v[h][want])


def brute_loop(q, k, chunk, budget, sinks, W, scale):
    """Explicit lists: cache = list of positions per head, rescored per chunk."""
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    g = Hq // Hkv
    caches = [[] for _ in range(Hkv)]
    for p0 in range(0, S, chunk):
        p1 = min(S, p0 + chunk)
        for h in range(Hkv):
            caches[h] += list(range(p0, p1))
        for h in range(Hkv):
            if len(caches[h]) <= budget:
                continue
            score = {}
            for t in caches[h]:
                terms = []
                for qh in range(h * g, (h + 1) * g):
                    for dq in range(max(p0, t + W), p1):
                        vis = [u for u in caches[h] if u <= dq]
                        logits = [math.fsum(q[qh][dq][c] * k[h][u][c] for c in range(d)) * scale
                                  for u in vis]
                        top = max(logits)
                        lse = top + math.log(math.fsum(math.exp(x - top) for x in logits))
                        terms.append(math.exp(logits[vis.index(t)] - lse))
                score[t] = math.fsum(terms)
            forced = [t for t in caches[h] if t < sinks or t >= p1 - W]
            cand = sorted((t for t in caches[h] if t not in forced), key=lambda t: (-score[t], t))
            n_keep = min(len(caches[h]), max(budget, len(forced)))
            caches[h] = sorted(forced + cand[:n_keep - len(forced)])
    return caches


@pytest.mark.parametrize("seed,S,C,budget,sinks,W", [(0, 30, 6, 10, 2, 3), (1, 26, 5, 8, 1, 2),
                                                      (2, 24, 8, 9, 2, 0)])
def test_loop_matches_brute_force(seed, S, C, budget, sinks, W):
    Hq, Hkv, d = 2, 1, 3
    q, k, v = rand(20 + seed, Hq, Hkv, S, d, spread=1.3)
    scale = 1 / math.sqrt(d)
    heads = ch.prefill_compress(q, k, v, C, budget, sinks, W, scale)
    want = brute_loop(q, k, C, budget, sinks, W, scale)
    for h in range(Hkv):
        assert heads[h].pos.tolist() == want[h]


def test_cache_invariants_after_every_compression():
    Hq, Hkv, S, d, C, budget, sinks, W = 4, 2, 150, 8, 24, 40, 4, 10
    q, k, v = rand(11, Hq, Hkv, S, d, spread=1.4)
    rec = []
    heads = ch.prefill_compress(q, k, v, C, budget, sinks, W, record=rec)
    for r in rec:
        n = r["pos"].shape[1]
        if r["kept_rows"] is None:
            assert n <= budget
            continue
        for h in range(Hkv):
            rows = r["kept_rows"][h]
            kept_pos = r["pos"][h][rows]
            assert rows.size == min(n, max(budget, sinks + W))
            assert np.all(np.diff(kept_pos) > 0)
            assert set(range(sinks)) <= set(kept_pos.tolist())
            assert set(range(r["p1"] - W, r["p1"])) <= set(kept_pos.tolist())
    for h in range(Hkv):
        np.testing.assert_array_equal(heads[h].k, k[h][heads[h].pos])
        np.testing.assert_array_equal(heads[h].v, v[h][heads[h].pos])


def test_planted_mistake_in_the_forced_window_is_caught():
    """A window forced as the last W+1 positions breaks the closed form."""
    S, C, budget, sinks, W = 100, 16, 30, 4, 8
    _, k, v = rand(9, 2, 2, S, 4)
    q = np.zeros((2, S, 4))
    orig = ch.compress_rows

    def wrong(mass, pos, budget, sinks, window, p_end):
        return orig(mass, pos, budget, sinks, window + 1, p_end)

    ch.compress_rows = wrong
    try:
        heads = ch.prefill_compress(q, k, v, C, budget, sinks, W)
    finally:
        ch.compress_rows = orig
    want = np.concatenate([np.arange(budget - W), np.arange(S - W, S)])
    assert not np.array_equal(heads[0].pos, want)
