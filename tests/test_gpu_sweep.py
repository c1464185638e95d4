"""A seeded sweep of random small shapes through the score passes, against the
fp64 oracle at the parity bar: |lse - ref| <= 1e-3, mass relative error
<= 2e-3 on every key with ref > 0, and exact zeros for keys no query counts.

The fixed cases elsewhere pick their shapes by hand; these draw them, so that
the boundaries of the kernels fall at many offsets at once:

* sequence lengths that are mostly not multiples of the 64-row tiles (the
  ragged last tile of both passes, whose rows are staged clamped);
* GQA ratios 1, 2, 3, 4 and 8, d = 64 and 128, bf16 and fp16, B = 1 and 2;
* windows from 0 to beyond S, so the mass pass's full and band steps and the
  first pass's causal diagonal split the tiles at every position;
* inputs that are contiguous, and inputs that are views into a wider
  [B, S, H, 2d] buffer (row stride H * 2d, base offset 0 or d elements).

Each case runs fam_compute and the per-query-head mass (each query head's
mass against the oracle's, and their group sums against the group mass to
fp32 rounding), the KVpop target epilogue on that mass (eps 0 or 1e-6, max
or mean over the group, against oracle.kvpop_target: 2.5e-3 absolute on the
log, -inf where the oracle has it), then the chunk mode on the same inputs:
the last Sq rows as the chunk's queries over all S keys, against the
oracle's chunk functions.

A second sweep draws eviction cases (head counts, lengths around the
4096-candidate chunks, sinks, windows, budgets from 0 past S, and scores that
are normal, heavy-tailed like masses, from a few distinct values, or mixed
with NaN, +-inf and +-0) and compares select bit for bit with the oracle's
sort-based selection, and compact (on cases up to 300000 rows) bit for bit
with its fancy-index gather.

A third draws ranking-quality cases (rows with ties and special values, head
counts and lengths around the 4096-entry tiles, budgets (s, w, k) of the
running cut-off from 0 past S): the rank order and the running cut-offs
exactly, the eviction cost to 1e-12 relative, against oracle/ranking.py and
oracle/topk_cutoff.py.
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam
from oracle import chunked as ch
from oracle import fam_oracle as fo
from oracle import kvpop_target as kt
from oracle import ranking as rk
from oracle import select_oracle as so
from oracle import topk_cutoff as tc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 1e-3
MASS_RTOL = 2e-3
TARGET_ATOL = 2.5e-3


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def to64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def check_lse(got, ref):
    err = np.abs(np.asarray(got, np.float64) - ref).max()
    assert err <= LSE_TOL, f"lse max abs err {err}"


def check_mass(got, ref):
    got = np.asarray(got, np.float64)
    assert np.all(got[ref == 0] == 0.0), "keys no query counts must be exactly 0"
    pos = ref > 0
    if pos.any():
        rel = np.abs(got[pos] - ref[pos]) / np.maximum(ref[pos], np.finfo(np.float32).tiny)
        assert rel.max() <= MASS_RTOL, f"mass max rel err {rel.max()}"


def check_target(got, ref):
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf positions differ"
    fin = np.isfinite(ref)
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= TARGET_ATOL, f"target max abs err {err}"


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        g = int(rng.choice([1, 2, 3, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        S = int(rng.integers(1, 900))
        W = int(rng.choice([0, int(rng.integers(0, 70)), int(rng.integers(0, S + 8))]))
        cases.append(dict(
            seed=1000 + i, B=int(rng.choice([1, 1, 2])), Hq=g * Hkv, Hkv=Hkv, S=S,
            d=int(rng.choice([64, 128])), W=W,
            dtype=torch.float16 if rng.random() < 0.3 else torch.bfloat16,
            layout=str(rng.choice(["contiguous", "view", "view+d"])),
            Sq=int(rng.integers(1, S + 1)), spread=float(rng.choice([0.7, 1.3]))))
    return cases


CASES = draw_cases(48, 20261202)


def inputs(c):
    """q [B, Hq, S, d] and k [B, Hkv, S, d] on the device, contiguous or as
    views into [B, S, H, 2d] buffers."""
    gen = torch.Generator().manual_seed(c["seed"])
    B, Hq, Hkv, S, d = c["B"], c["Hq"], c["Hkv"], c["S"], c["d"]
    if c["layout"] == "contiguous":
        q = (torch.randn(B, Hq, S, d, generator=gen) * c["spread"]).to(c["dtype"]).to(DEV)
        k = (torch.randn(B, Hkv, S, d, generator=gen) * c["spread"]).to(c["dtype"]).to(DEV)
        return q, k
    off = d if c["layout"] == "view+d" else 0
    qb = (torch.randn(B, S, Hq, 2 * d, generator=gen) * c["spread"]).to(c["dtype"]).to(DEV)
    kb = (torch.randn(B, S, Hkv, 2 * d, generator=gen) * c["spread"]).to(c["dtype"]).to(DEV)
    q = qb[..., off:off + d].permute(0, 2, 1, 3)
    k = kb[..., off:off + d].permute(0, 2, 1, 3)
    assert q.stride(3) == 1 and q.stride(2) == Hq * 2 * d
    return q, k


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"s{c['seed']}")
def test_random_shape_against_oracle(c):
    B, Hq, Hkv, S, d, W, Sq = c["B"], c["Hq"], c["Hkv"], c["S"], c["d"], c["W"], c["Sq"]
    say(f"sweep seed={c['seed']} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W} Sq={Sq} "
        f"{c['dtype']} {c['layout']} spread={c['spread']}")
    q, k = inputs(c)
    lse, mass = fam.fam_compute(q, k, W)
    mass_q = fam.fam_mass_per_head(q, k, lse, W)
    eps = (0.0, 1e-6)[c["seed"] % 2]
    agg = ("max", "mean")[(c["seed"] // 2) % 2]
    tgt = fam.fam_kvpop_target(mass_q, Hkv, W, eps=eps, aggregate=agg)
    lse_c, mass_c = fam.fam_compute_chunk(q[:, :, S - Sq:], k, W)
    torch.cuda.synchronize()
    qn, kn = to64(q), to64(k)
    pos = np.tile(np.arange(S, dtype=np.int64), (Hkv, 1))
    for b in range(B):
        lse_ref = fo.causal_lse(qn[b], kn[b])
        mass_ref, per_q_ref = fo.future_mass(qn[b], kn[b], lse_ref, W, per_query_head=True)
        check_lse(to64(lse[b]), lse_ref)
        check_mass(to64(mass[b]), mass_ref)
        check_mass(to64(mass_q[b]), per_q_ref)
        g = Hq // Hkv
        for h in range(Hkv):
            check_target(to64(tgt[b, h]), kt.target(per_q_ref[h * g:(h + 1) * g], W, eps=eps, aggregate=agg))
        lse_cref = ch.chunk_lse(qn[b, :, S - Sq:], kn[b], pos, S - Sq)
        mass_cref = ch.chunk_mass(qn[b, :, S - Sq:], kn[b], pos, lse_cref, S - Sq, W)
        check_lse(to64(lse_c[b]), lse_cref)
        check_mass(to64(mass_c[b]), mass_cref)
    grp = mass_q.view(B, Hkv, Hq // Hkv, S).double().sum(2)
    np.testing.assert_allclose(grp.cpu().numpy(), to64(mass), rtol=1e-5, atol=0)


def draw_select_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.choice([int(rng.integers(1, 600)), int(rng.integers(3000, 9000)),
                            int(rng.integers(9000, 40000))]))
        cases.append(dict(seed=2000 + i, H=int(rng.integers(1, 70)), S=S,
                          sinks=int(rng.choice([0, 1, 4, int(rng.integers(0, 50))])),
                          recent=int(rng.choice([0, 16, 512, int(rng.integers(0, 300))])),
                          kind=str(rng.choice(["normal", "heavy", "few", "special"]))))
    return cases


SELECT_CASES = draw_select_cases(40, 20261203)


def select_scores(rng, kind, H, S):
    if kind == "normal":
        return rng.standard_normal((H, S)).astype(np.float32)
    if kind == "heavy":                       # positive, spanning many octaves, like masses
        return np.exp(rng.standard_normal((H, S)) * 4.0).astype(np.float32)
    if kind == "few":                         # many equal keys: ties go to the lower position
        return rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=(H, S))
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5, 1e-38], np.float32)
    s = rng.choice(pool, size=(H, S)).astype(np.float32)
    mix = rng.random((H, S)) < 0.5
    s[mix] = rng.standard_normal(mix.sum()).astype(np.float32)
    return s


@pytest.mark.parametrize("c", SELECT_CASES, ids=lambda c: f"s{c['seed']}")
def test_random_select_and_compact_against_oracle(c):
    H, S, sinks, recent = c["H"], c["S"], c["sinks"], c["recent"]
    say(f"select sweep seed={c['seed']} H={H} S={S} sinks={sinks} recent={recent} {c['kind']}")
    rng = np.random.default_rng(c["seed"])
    scores = select_scores(rng, c["kind"], H, S)
    budgets = [int(x) for x in rng.integers(0, S + 8, H)]
    idx, off = fam.evict_select(torch.from_numpy(scores).to(DEV), budgets, sinks, recent)
    torch.cuda.synchronize()
    idx_ref, off_ref = so.select(scores, budgets, sinks, recent)
    assert off.cpu().numpy().tolist() == off_ref.tolist()
    assert np.array_equal(idx.cpu().numpy(), idx_ref), "index lists differ"
    if H * S <= 300000:   # the gather too (K/V of d = 64 as raw 16-bit patterns)
        kv = torch.from_numpy(rng.integers(-30000, 30000, size=(2, H, S, 64), dtype=np.int16))
        k_new, v_new = fam.kv_compact(kv[0].view(torch.bfloat16).to(DEV), kv[1].view(torch.bfloat16).to(DEV),
                                      idx, off)
        torch.cuda.synchronize()
        assert np.array_equal(k_new.cpu().view(torch.int16).numpy(), so.compact(kv[0].numpy(), idx_ref, off_ref))
        assert np.array_equal(v_new.cpu().view(torch.int16).numpy(), so.compact(kv[1].numpy(), idx_ref, off_ref))


def draw_ranking_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(1000, 9000)),
                            int(rng.integers(9000, 20000))]))
        cases.append(dict(seed=3000 + i, H=int(rng.integers(1, 12)), S=S,
                          s=int(rng.choice([0, 1, 4, int(rng.integers(0, S + 4))])),
                          w=int(rng.choice([0, 3, 512, int(rng.integers(0, S + 4))])),
                          k=int(rng.choice([0, 1, int(rng.integers(0, S + 4))]))))
    return cases


RANKING_CASES = draw_ranking_cases(32, 20261204)


@pytest.mark.parametrize("c", RANKING_CASES, ids=lambda c: f"s{c['seed']}")
def test_random_ranking_and_cutoffs_against_oracle(c):
    H, S, s, w, k = c["H"], c["S"], c["s"], c["w"], c["k"]
    say(f"ranking sweep seed={c['seed']} H={H} S={S} s={s} w={w} k={k}")
    rng = np.random.default_rng(c["seed"])
    scores = rng.standard_normal((H, S)).astype(np.float32)
    scores[rng.random((H, S)) < 0.1] = 0.5                  # ties
    scores[rng.random((H, S)) < 0.02] = np.nan
    scores[rng.random((H, S)) < 0.02] = -0.0
    imp = (rng.random((H, S)) ** 3).astype(np.float32)
    sd, impd = torch.from_numpy(scores).to(DEV), torch.from_numpy(imp).to(DEV)
    order = fam.fam_rank_order(sd)
    cost = fam.fam_eviction_cost(impd, order)
    cut = fam.fam_topk_cutoff(order, s, w, k)
    torch.cuda.synchronize()
    order_ref = rk.rank_order(scores)
    np.testing.assert_array_equal(order.cpu().numpy(), order_ref)
    np.testing.assert_allclose(cost.cpu().numpy(), rk.eviction_cost(imp.astype(np.float64), order_ref),
                               rtol=1e-12, atol=0)
    got = cut.cpu().numpy()
    for h in range(H):
        ranks = tc.ranks_from_scores(scores[h].astype(np.float64))
        np.testing.assert_array_equal(got[h], tc.cutoffs(ranks, s, w, k))
