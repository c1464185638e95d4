"""GPU parity of the ranking-quality measures against oracle/ranking.py.

fam_rank_order must equal the oracle's order exactly (ties to the lower
position, NaN last, -0.0 equal to +0.0), on rows with ties, specials, ragged
lengths and the 128k workload's masses. fam_eviction_cost is an fp64 sum of
(r + 1) * importance and must match the oracle's sum over budgets to 1e-12
relative. fam_retention_overlap counts are exact. The normalised cost is 1
exactly for the optimal order and at least 1 otherwise.
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads
from oracle import ranking as rk
from oracle import select_oracle as so

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def special_rows(seed, H, n):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((H, n)).astype(np.float32)
    s[rng.random((H, n)) < 0.1] = 0.5                 # ties
    s[rng.random((H, n)) < 0.02] = np.nan
    s[rng.random((H, n)) < 0.02] = -0.0
    s[rng.random((H, n)) < 0.02] = 0.0
    s[rng.random((H, n)) < 0.01] = np.inf
    s[rng.random((H, n)) < 0.01] = -np.inf
    return s


@pytest.mark.parametrize("seed,H,n", [(1, 1, 1), (2, 3, 1000), (3, 2, 1025), (4, 10, 4097),
                                      (5, 1, 70001), (6, 8, 3000),
                                      # up to 64 tiles of 4096 the place launch forms its own
                                      # digit slots; beyond, a scan launch does
                                      (10, 2, 262144), (11, 2, 262145), (12, 1, 300007)])
def test_rank_order_matches_oracle(seed, H, n):
    say(f"fam_rank_order seed={seed} H={H} n={n}")
    s = special_rows(seed, H, n)
    got = fam.fam_rank_order(torch.from_numpy(s).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, rk.rank_order(s))


def test_rank_order_all_equal_and_strided_rows():
    say("fam_rank_order all-equal rows and a strided view")
    s = torch.zeros(3, 5000, device=DEV)
    np.testing.assert_array_equal(fam.fam_rank_order(s).cpu().numpy(), np.tile(np.arange(5000), (3, 1)))
    big = torch.randn(4, 3000, generator=torch.Generator().manual_seed(1)).to(DEV)
    view = big[:, 100:2100]
    got = fam.fam_rank_order(view).cpu().numpy()
    np.testing.assert_array_equal(got, rk.rank_order(view.cpu().numpy()))


@pytest.mark.parametrize("seed,H,n", [(7, 2, 1), (8, 4, 2000), (9, 8, 20000)])
def test_eviction_cost_matches_oracle(seed, H, n):
    say(f"fam_eviction_cost seed={seed} H={H} n={n}")
    rng = np.random.default_rng(seed)
    imp = (rng.random((H, n)) ** 3).astype(np.float32)
    s = rng.standard_normal((H, n)).astype(np.float32)
    impd, sd = torch.from_numpy(imp).to(DEV), torch.from_numpy(s).to(DEV)
    for scores in (s, imp, -imp):
        order = fam.fam_rank_order(torch.from_numpy(scores).to(DEV))
        got = fam.fam_eviction_cost(impd, order).cpu().numpy()
        ref = rk.eviction_cost(imp.astype(np.float64), rk.rank_order(scores))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)
    ratio = fam.eviction_cost_ratio(sd, impd).cpu().numpy()
    np.testing.assert_allclose(ratio, rk.normalized_cost(s, imp.astype(np.float64)), rtol=1e-12)
    assert np.all(ratio >= 1.0)
    assert np.all(fam.eviction_cost_ratio(impd, impd).cpu().numpy() == 1.0)


def test_cost_ratio_in_library_against_oracle_and_costs():
    """fam_eviction_cost_ratio against the oracle's normalised cost, against
    the quotient of the two fam_eviction_cost results (bit for bit, the same
    sums), on strided rows, and 1 for heads without importance."""
    say("fam_eviction_cost_ratio")
    H, n = 6, 9000
    rng = np.random.default_rng(21)
    imp = (rng.random((H, n)) ** 4).astype(np.float32)
    imp[2] = 0.0                                         # no importance: ratio 1
    imp[4] = 0.0
    imp[4, 123] = 2.5                                    # importance on one entry
    s = rng.standard_normal((H, n)).astype(np.float32)
    s[:, rng.random(n) < 0.05] = 0.5                     # ties
    big = torch.from_numpy(np.concatenate([s, imp], axis=1)).to(DEV)    # strided rows of both
    sd, impd = big[:, :n], big[:, n:]
    ratio = fam.fam_eviction_cost_ratio(sd, impd).cpu().numpy()
    ref = rk.normalized_cost(s.astype(np.float64), imp.astype(np.float64))
    np.testing.assert_allclose(ratio, ref, rtol=1e-12)
    assert ratio[2] == 1.0
    c = fam.fam_eviction_cost(impd.contiguous(), fam.fam_rank_order(sd.contiguous())).cpu().numpy()
    c_opt = fam.fam_eviction_cost(impd.contiguous(), fam.fam_rank_order(impd.contiguous())).cpu().numpy()
    live = c_opt != 0
    assert np.array_equal(ratio[live], c[live] / c_opt[live])
    assert np.all(ratio >= 1.0)


def test_retention_overlap_on_selections():
    say("fam_retention_overlap of two evict_select outputs")
    H, S = 8, 20000
    g = torch.Generator().manual_seed(3)
    a_scores = torch.rand(H, S, generator=g)
    b_scores = a_scores + 0.3 * torch.rand(H, S, generator=g)
    budgets = [100, 5000, 20000, 0, 300, 7000, 1, 12345]
    ia, oa = fam.evict_select(a_scores.to(DEV), budgets, 4, 64)
    ib, ob = fam.evict_select(b_scores.to(DEV), budgets, 4, 64)
    got = fam.fam_retention_overlap(ia, oa, ib, ob, S).cpu().numpy()
    ia_h, oa_h, ib_h, ob_h = ia.cpu().numpy(), oa.cpu().numpy(), ib.cpu().numpy(), ob.cpu().numpy()
    for h in range(H):
        a = ia_h[oa_h[h]:oa_h[h + 1]]
        b = ib_h[ob_h[h]:ob_h[h + 1]]
        assert got[h] == len(set(a.tolist()) & set(b.tolist()))
        assert got[h] / len(a) == rk.retention_recall(a, b)


def test_retention_overlap_at_300000_positions_eight_heads():
    """Beyond one 262144-position bitmap: the selections of two scorers over
    8 heads of 300000 positions (the round-based select path), counted in
    two windows, against set arithmetic; lists with positions on both sides
    of the window edge and duplicates."""
    say("fam_retention_overlap S=300000 H=8")
    H, S = 8, 300000
    rng = np.random.default_rng(17)
    a_scores = rng.exponential(size=(H, S)).astype(np.float32)
    b_scores = (a_scores + 0.5 * rng.random((H, S))).astype(np.float32)
    budgets = [int(x) for x in rng.integers(1000, S, H)]
    ia, oa = fam.evict_select(torch.from_numpy(a_scores).to(DEV), budgets, 4, 512)
    ib, ob = fam.evict_select(torch.from_numpy(b_scores).to(DEV), budgets, 4, 512)
    got = fam.fam_retention_overlap(ia, oa, ib, ob, S).cpu().numpy()
    ia_h, oa_h, ib_h, ob_h = ia.cpu().numpy(), oa.cpu().numpy(), ib.cpu().numpy(), ob.cpu().numpy()
    for h in range(H):
        a = ia_h[oa_h[h]:oa_h[h + 1]]
        b = ib_h[ob_h[h]:ob_h[h + 1]]
        assert got[h] == len(set(a.tolist()) & set(b.tolist())), h
    edge = 1 << 18
    a = torch.tensor([edge - 1, edge, edge, S - 1, 5, -3], dtype=torch.int32, device=DEV)
    b = torch.tensor([edge, edge - 1, S - 1, S - 1, S, 5, edge + 1], dtype=torch.int32, device=DEV)
    oa1 = torch.tensor([0, 6], dtype=torch.int64, device=DEV)
    ob1 = torch.tensor([0, 7], dtype=torch.int64, device=DEV)
    assert fam.fam_retention_overlap(a, oa1, b, ob1, S).cpu().tolist() == [4]


def test_retention_overlap_duplicates_and_out_of_range():
    say("fam_retention_overlap hand cases")
    a = torch.tensor([1, 2, 3, 3, 9, 0, 5], dtype=torch.int32, device=DEV)
    oa = torch.tensor([0, 5, 5, 7], dtype=torch.int64, device=DEV)
    b = torch.tensor([3, 3, 2, 99, -1, 7, 0, 5, 5], dtype=torch.int32, device=DEV)
    ob = torch.tensor([0, 5, 6, 9], dtype=torch.int64, device=DEV)
    got = fam.fam_retention_overlap(a, oa, b, ob, 10).cpu().tolist()
    assert got == [2, 0, 2]


def test_llama_128k_ranking_of_recency_against_mass():
    """At full size: rank the 128k layer's masses (the teacher) and a recency
    score (newest first); orders and costs against the oracle for two heads,
    recall of the recency kept set against the mass kept set."""
    wl = workloads.llama31_8b_128k()
    say(wl.name)
    t = wl.tensors(with_v=False)
    q, k = t["q"].to(DEV), t["k"].to(DEV)
    _, mass = fam.fam_compute(q, k, wl.W)
    del q, k
    m = mass[0]
    H, S = m.shape
    recency = torch.arange(S, dtype=torch.float32, device=DEV).expand(H, S).contiguous()
    order_m = fam.fam_rank_order(m)
    order_r = fam.fam_rank_order(recency)
    ratio = fam.eviction_cost_ratio(recency, m).cpu().numpy()
    assert np.all(ratio > 1.0)
    mh = m.cpu().numpy()
    for h in (0, 5):
        np.testing.assert_array_equal(order_m[h].cpu().numpy(), rk.rank_order(mh[h:h + 1])[0])
        ref = rk.normalized_cost(np.arange(S)[None].astype(np.float64), mh[h:h + 1].astype(np.float64))
        np.testing.assert_allclose(ratio[h], ref[0], rtol=1e-12)
    assert np.array_equal(order_r[0].cpu().numpy(), np.arange(S)[::-1])
    budgets = [S // 8] * H
    ia, oa = fam.evict_select(m, budgets, wl.sinks, wl.recent)
    ib, ob = fam.evict_select(recency, budgets, wl.sinks, wl.recent)
    common = fam.fam_retention_overlap(ia, oa, ib, ob, S).cpu().numpy()
    ia_h, ib_h = ia.cpu().numpy().reshape(H, -1), ib.cpu().numpy().reshape(H, -1)
    for h in range(H):
        assert common[h] == len(set(ia_h[h].tolist()) & set(ib_h[h].tolist()))
