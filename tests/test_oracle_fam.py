"""Pins for the fp64 future-attention-mass oracle (CPU only).

The oracle is checked against things other than itself:
  * brute force written as pure-Python loops with math.fsum (tiny sizes),
  * the W = 0 invariant (each causal softmax row sums to one, so the column
    masses of a KV head sum to S * g),
  * the uniform-logit closed form (harmonic numbers),
  * the single-sink closed form,
  * the S = 1 special case,
and each pin is shown to reject a plausible mistake (an off-by-one window,
a dropped diagonal, a wrong GQA mapping, a transposed operand).
"""
import math

import numpy as np
import pytest

from oracle import fam_oracle as fo


def brute(q, k, W, scale):
    """Pure-Python reference: q [Hq,S,d], k [Hkv,S,d] as nested lists."""
    Hq, S, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k)
    g = Hq // Hkv
    logit = [[[math.fsum(q[qh][i][c] * k[qh // g][j][c] for c in range(d)) * scale
               for j in range(i + 1)] for i in range(S)] for qh in range(Hq)]
    lse = []
    for qh in range(Hq):
        row = []
        for i in range(S):
            top = max(logit[qh][i])
            row.append(top + math.log(math.fsum(math.exp(x - top) for x in logit[qh][i])))
        lse.append(row)
    mass = []
    for h in range(Hkv):
        col = []
        for j in range(S):
            terms = [math.exp(logit[qh][i][j] - lse[qh][i])
                     for qh in range(h * g, (h + 1) * g) for i in range(j + W, S)]
            col.append(math.fsum(terms))
        mass.append(col)
    return np.array(lse), np.array(mass)


def rand_qk(seed, Hq, Hkv, S, d, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, S, d)) * spread
    k = rng.standard_normal((Hkv, S, d)) * spread
    return q, k


CASES = [
    # (seed, Hq, Hkv, S, d, W)
    (0, 1, 1, 17, 4, 0), (1, 2, 1, 23, 4, 3), (2, 4, 1, 31, 4, 1),
    (3, 4, 2, 40, 4, 39), (4, 2, 2, 33, 64, 5), (5, 4, 2, 64, 4, 64),
    (6, 4, 1, 29, 4, 100), (7, 1, 1, 1, 4, 0), (8, 2, 1, 2, 64, 1),
]


@pytest.mark.parametrize("seed,Hq,Hkv,S,d,W", CASES)
def test_oracle_matches_brute_force(seed, Hq, Hkv, S, d, W):
    q, k = rand_qk(seed, Hq, Hkv, S, d, spread=1.5)
    scale = 1.0 / math.sqrt(d)
    lse_b, mass_b = brute(q.tolist(), k.tolist(), W, scale)
    lse, mass = fo.fam(q, k, W, block=7)
    np.testing.assert_allclose(lse, lse_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mass, mass_b, rtol=1e-11, atol=1e-14)


def test_brute_force_rejects_off_by_one_window():
    q, k = rand_qk(11, 2, 1, 20, 4)
    lse_b, mass_b = brute(q.tolist(), k.tolist(), 3, 0.5)
    lse = fo.causal_lse(q, k, 0.5)
    wrong = fo.future_mass(q, k, lse, 4, 0.5)      # i > j + W instead of >=
    assert np.abs(wrong - mass_b).max() > 1e-3


def test_brute_force_rejects_wrong_gqa_mapping():
    q, k = rand_qk(12, 4, 2, 16, 4)
    lse_b, _ = brute(q.tolist(), k.tolist(), 0, 0.5)
    # interleaved mapping qh -> qh % Hkv instead of contiguous groups
    lse_wrong = fo.causal_lse(q, k[[0, 1, 0, 1]], 0.5)
    lse_right = fo.causal_lse(q, k[[0, 0, 1, 1]], 0.5)
    np.testing.assert_allclose(lse_right, lse_b, atol=1e-12)
    assert np.abs(lse_wrong - lse_b).max() > 1e-3


@pytest.mark.parametrize("seed,Hq,Hkv,S,d", [(20, 4, 1, 300, 16), (21, 8, 2, 257, 64),
                                             (22, 2, 2, 1, 8), (23, 6, 3, 129, 32)])
def test_w0_columns_sum_to_rows(seed, Hq, Hkv, S, d):
    q, k = rand_qk(seed, Hq, Hkv, S, d, spread=2.0)
    lse, mass = fo.fam(q, k, 0, block=64)
    g = Hq // Hkv
    np.testing.assert_allclose(mass.sum(axis=1), np.full(Hkv, S * g), rtol=1e-12)


def test_w0_invariant_rejects_dropped_diagonal():
    q, k = rand_qk(24, 2, 1, 50, 8)
    lse, _ = fo.fam(q, k, 0)
    # a normaliser that forgets the key j = i makes rows sum above one
    logit = (q[0] @ k[0].T) / math.sqrt(8)
    strict = np.array([np.log(np.exp(logit[i, :i]).sum()) if i else 0.0 for i in range(50)])
    assert abs(lse[0] - strict).max() > 1e-3


def harmonic(n):
    return math.fsum(1.0 / m for m in range(1, n + 1))


@pytest.mark.parametrize("Hq,Hkv,S,W", [(2, 1, 200, 0), (4, 2, 311, 7), (1, 1, 64, 63), (4, 4, 50, 80)])
def test_uniform_logits_closed_form(Hq, Hkv, S, W):
    rng = np.random.default_rng(S)
    d = 8
    q = np.zeros((Hq, S, d))
    k = rng.standard_normal((Hkv, S, d))
    lse, mass = fo.fam(q, k, W, block=37)
    g = Hq // Hkv
    np.testing.assert_allclose(lse, np.log(np.arange(1, S + 1))[None, :].repeat(Hq, 0), rtol=0, atol=1e-13)
    expect = np.array([g * (harmonic(S) - harmonic(j + W)) if j <= S - 1 - W else 0.0 for j in range(S)])
    np.testing.assert_allclose(mass, expect[None, :].repeat(Hkv, 0), rtol=1e-12, atol=1e-15)


def test_equal_key_rows_closed_form():
    # all keys of the head equal: each row's logits are equal, same closed form
    rng = np.random.default_rng(5)
    S, d, W = 120, 16, 9
    q = rng.standard_normal((2, S, d))
    k = np.repeat(rng.standard_normal((1, 1, d)), S, axis=1)
    lse, mass = fo.fam(q, k, W)
    logit_i = (q[:, :, :] @ k[0, 0]) / math.sqrt(d)
    np.testing.assert_allclose(lse, logit_i + np.log(np.arange(1, S + 1))[None, :], atol=1e-12)
    expect = np.array([2 * (harmonic(S) - harmonic(j + W)) if j <= S - 1 - W else 0.0 for j in range(S)])
    np.testing.assert_allclose(mass[0], expect, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("a,b,W,S,g", [(4.0, 2.0, 3, 90, 2), (8.0, 4.0, 0, 70, 1), (2.0, 0.5, 12, 64, 4)])
def test_single_sink_closed_form(a, b, W, S, g):
    d = 16
    scale = 1.0 / math.sqrt(d)
    q = np.zeros((g, S, d))
    q[:, :, 0] = a
    k = np.zeros((1, S, d))
    k[0, 0, 0] = b
    lse, mass = fo.fam(q, k, W, block=19)
    ec = math.exp(a * b * scale)
    np.testing.assert_allclose(lse, np.log(ec + np.arange(S))[None, :].repeat(g, 0), atol=1e-12)
    expect = np.zeros(S)
    expect[0] = g * math.fsum(ec / (ec + i) for i in range(W, S))
    for j in range(1, S):
        expect[j] = g * math.fsum(1.0 / (ec + i) for i in range(j + W, S))
    np.testing.assert_allclose(mass[0], expect, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("W,expect", [(0, 3.0), (1, 0.0), (5, 0.0)])
def test_single_token(W, expect):
    q = np.array([[[0.5, -1.0]]] * 3)
    k = np.array([[[2.0, 0.25]]])
    lse, mass = fo.fam(q, k, W)
    np.testing.assert_allclose(lse, np.full((3, 1), (0.5 * 2.0 - 0.25) / math.sqrt(2)), atol=1e-15)
    assert mass[0, 0] == pytest.approx(expect, abs=1e-15)


def test_transposed_operand_is_caught():
    # swapping q and k (a transposed-pass bookkeeping slip) changes the result
    q, k = rand_qk(30, 1, 1, 40, 8)
    lse_b, mass_b = brute(q.tolist(), k.tolist(), 2, 0.3)
    _, mass_swapped = fo.fam(k, q, 2, scale=0.3)
    assert np.abs(mass_swapped - mass_b).max() > 1e-3


def test_tail_keys_helper_matches_full_mass():
    q, k = rand_qk(31, 4, 2, 96, 8)
    W = 10
    lse, mass = fo.fam(q, k, W)
    tail = 60
    keys = np.arange(tail - W, 96)
    for h in range(2):
        got = fo.future_mass_keys(q[2 * h:2 * h + 2], k[h], lse[2 * h:2 * h + 2, tail:], tail, keys, W)
        np.testing.assert_allclose(got, mass[h, keys], rtol=1e-12, atol=1e-15)


def test_lse_rows_helper_matches_full():
    q, k = rand_qk(32, 2, 1, 80, 8)
    lse = fo.causal_lse(q, k)
    rows = np.array([0, 1, 37, 79])
    np.testing.assert_allclose(fo.causal_lse_rows(q[1], k[0], rows, 1 / math.sqrt(8)), lse[1, rows], atol=1e-13)
