"""GPU tests of fam_mass_select (bit-exact).

The call's masses, index lists and offsets must equal, bit for bit, those of
fam_mass followed by evict_select on the same inputs, whether it takes the
fused path (the launch that adds the mass pass's partial sums also builds the
selection's first histograms) or runs the two steps one after the other; the
index lists must also equal the oracle's selection on the returned masses.
Cases cover the short-sequence splits, the ranges of query rows from 65536
keys on, rows whose length is not a multiple of 4, positions before the first
and after the last chunk, and every fallback (no split, one chunk a head,
trivial budgets, more heads than one batch, more candidates than the
three-launch select takes).
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads
from oracle import select_oracle as so

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def inputs(seed, B, Hq, Hkv, S, d=128, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, S, d, generator=g).to(dtype).to(DEV)
    k = torch.randn(B, Hkv, S, d, generator=g).to(dtype).to(DEV)
    return q, k


def budgets_for(seed, H, S, sinks, recent):
    """Per-head budgets between the forced set and S, with one head that keeps
    only its forced rows when there are several heads."""
    rng = np.random.default_rng(seed)
    forced = min(S, min(sinks, S) + max(0, min(recent, S - min(sinks, S))))
    b = [int(x) for x in rng.integers(forced + 1, S + 1, H)]
    if H > 1:
        b[-1] = 0
    return b


def check(q, k, W, budgets, sinks, recent, mass_ws_bytes=None):
    """fam_mass_select against fam_mass + evict_select and the oracle."""
    B, Hq, S, _ = q.shape
    Hkv = k.shape[1]
    lse = fam.fam_lse(q, k)
    mws = None
    if mass_ws_bytes is not None:
        mws = torch.empty(max(mass_ws_bytes, 16), dtype=torch.uint8, device=DEV)
    mass, idx, off = fam.fam_mass_select(q, k, lse, W, budgets, sinks, recent, mass_workspace=mws)
    ref_mass = fam.fam_mass(q, k, lse, W, workspace=mws)
    ref_idx, ref_off = fam.evict_select(ref_mass.reshape(B * Hkv, S), budgets, sinks, recent)
    torch.cuda.synchronize()
    assert torch.equal(mass.view(torch.int32), ref_mass.view(torch.int32)), "masses differ"
    assert torch.equal(off, ref_off), "offsets differ"
    assert torch.equal(idx, ref_idx), "index lists differ"
    o_idx, o_off = so.select(mass.reshape(B * Hkv, S).cpu().numpy(), budgets, sinks, recent)
    assert off.cpu().numpy().tolist() == o_off.tolist()
    assert np.array_equal(idx.cpu().numpy(), o_idx), "index lists differ from the oracle's"
    return mass, idx, off


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,W,sinks,recent", [
    (1, 1, 8, 2, 9001, 64, 4, 64),        # rows not a multiple of 4: no 16-byte loads
    (2, 2, 4, 2, 12288, 16, 7, 5000),     # positions before the first and after the last chunk
    (3, 1, 4, 4, 8192, 0, 0, 0),          # no sinks, no window
    (4, 1, 8, 8, 16384, 128, 4, 128),     # eight heads, one a XCD
    (5, 1, 6, 3, 70001, 512, 4, 512),     # ranges of query rows, ragged rows
    (6, 3, 8, 4, 8200, 32, 4, 32),        # 12 heads: a last group of 8 heads only half full
    (7, 8, 8, 8, 8192, 16, 4, 16),        # 64 heads: one full batch
])
def test_mass_select_matches_two_calls(seed, B, Hq, Hkv, S, W, sinks, recent):
    say(f"fam_mass_select seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} W={W} sinks={sinks} recent={recent}")
    assert fam.fam_mass_workspace_size(B, Hq, Hkv, S) > 0
    q, k = inputs(seed, B, Hq, Hkv, S)
    check(q, k, W, budgets_for(seed, B * Hkv, S, sinks, recent), sinks, recent)


@pytest.mark.parametrize("name", ["tiny", "qwen3_4b", "long_trace", "llama_128k"])
def test_mass_select_on_workloads(name):
    wl = {"tiny": workloads.tiny, "qwen3_4b": workloads.qwen3_4b_layer, "long_trace": workloads.long_trace,
          "llama_128k": workloads.llama31_8b_128k}[name]()
    say(f"fam_mass_select {wl.name}")
    t = wl.tensors(with_v=False)
    q, k = t["q"].to(DEV), t["k"].to(DEV)
    bi = wl.budget_inputs()
    budgets = (so.budgets_from_ratios(bi["ratios"], bi["t"]).tolist() if "ratios" in bi
               else [bi["uniform"]] * wl.Hkv)
    mass, idx, off = check(q, k, wl.W, budgets, wl.sinks, wl.recent)
    if name == "llama_128k":   # the fused path twice: the same bits
        lse = fam.fam_lse(q, k)
        m2, i2, o2 = fam.fam_mass_select(q, k, lse, wl.W, budgets, wl.sinks, wl.recent)
        torch.cuda.synchronize()
        assert torch.equal(m2.view(torch.int32), mass.view(torch.int32))
        assert torch.equal(i2, idx) and torch.equal(o2, off)


def test_mass_select_fallbacks():
    """Paths that run the two steps in sequence give the same results."""
    say("fam_mass_select fallbacks")
    q, k = inputs(11, 1, 4, 2, 8192)
    # no split (a workspace too small for one): the mass pass reduces nothing
    check(q, k, 32, budgets_for(11, 2, 8192, 4, 32), 4, 32, mass_ws_bytes=16)
    # every head trivial: all candidates or none
    check(q, k, 32, [8192, 0], 4, 32)
    # one chunk a head
    q1, k1 = inputs(12, 1, 4, 2, 4000)
    check(q1, k1, 32, budgets_for(12, 2, 4000, 4, 32), 4, 32)
    # more heads than one select batch (72 > 64)
    q2, k2 = inputs(13, 9, 8, 8, 5000, d=64)
    check(q2, k2, 16, budgets_for(13, 72, 5000, 4, 16), 4, 16)
    # more than 131072 candidates a head: the round-based select after the mass pass's ranges
    q3, k3 = inputs(14, 1, 2, 1, 140000, d=64)
    check(q3, k3, 256, [50000], 4, 256)


def test_mass_select_fp16_and_strided_views():
    say("fam_mass_select fp16, transposed views")
    q, k = inputs(21, 1, 4, 2, 10000, dtype=torch.float16)
    check(q, k, 100, budgets_for(21, 2, 10000, 4, 100), 4, 100)
    # [B, S, H, d] storage seen as [B, H, S, d]
    g = torch.Generator().manual_seed(22)
    qs = torch.randn(1, 10000, 4, 128, generator=g).to(torch.bfloat16).to(DEV).transpose(1, 2)
    ks = torch.randn(1, 10000, 2, 128, generator=g).to(torch.bfloat16).to(DEV).transpose(1, 2)
    check(qs, ks, 100, budgets_for(22, 2, 10000, 4, 100), 4, 100)


def check_prepared(q, k, W, budget_sets, sinks, recent, mass_ws_bytes=None):
    """fam_mass_prepare_select, then evict_select_prepared with each budget set
    on the one prepared workspace, against fam_mass + evict_select and the
    oracle."""
    B, Hq, S, _ = q.shape
    Hkv = k.shape[1]
    lse = fam.fam_lse(q, k)
    mws = None
    if mass_ws_bytes is not None:
        mws = torch.empty(max(mass_ws_bytes, 16), dtype=torch.uint8, device=DEV)
    mass, sws = fam.fam_mass_prepare_select(q, k, lse, W, sinks, recent, mass_workspace=mws)
    ref_mass = fam.fam_mass(q, k, lse, W, workspace=mws)
    torch.cuda.synchronize()
    assert torch.equal(mass.view(torch.int32), ref_mass.view(torch.int32)), "masses differ"
    rows = mass.reshape(B * Hkv, S)
    for budgets in budget_sets:
        idx, off = fam.evict_select_prepared(rows, budgets, sinks, recent, sws)
        ref_idx, ref_off = fam.evict_select(rows, budgets, sinks, recent)
        torch.cuda.synchronize()
        assert torch.equal(off, ref_off), f"offsets differ for budgets {budgets}"
        assert torch.equal(idx, ref_idx), f"index lists differ for budgets {budgets}"
        o_idx, o_off = so.select(rows.cpu().numpy(), budgets, sinks, recent)
        assert np.array_equal(idx.cpu().numpy(), o_idx), "index lists differ from the oracle's"


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,W,sinks,recent,split", [
    (11, 1, 8, 2, 9001, 64, 4, 64, True),      # split mass pass: histograms in its reduction
    (12, 1, 8, 2, 9001, 64, 4, 64, False),     # no split: a histogram launch of its own
    (13, 2, 4, 2, 12288, 16, 7, 5000, True),   # positions before the first and after the last chunk
    (14, 1, 6, 3, 70001, 512, 4, 512, True),   # ranges of query rows, ragged rows
    (15, 8, 8, 8, 8192, 16, 4, 16, True),      # 64 heads: one full batch
    (16, 1, 4, 2, 4000, 16, 4, 16, True),      # one chunk a head: nothing prepared
    (17, 9, 8, 8, 8192, 16, 4, 16, True),      # 72 heads, more than one batch: nothing prepared
])
def test_prepared_select_matches_two_calls(seed, B, Hq, Hkv, S, W, sinks, recent, split):
    say(f"fam_mass_prepare_select seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} W={W} split={split}")
    q, k = inputs(seed, B, Hq, Hkv, S)
    H = B * Hkv
    forced = min(S, sinks + min(recent, max(0, S - sinks)))
    sets = [budgets_for(seed, H, S, sinks, recent),
            [forced] * H,                                   # every head trivial: the last launch alone
            [S] * H,
            budgets_for(seed + 100, H, S, sinks, recent)]
    check_prepared(q, k, W, sets, sinks, recent, None if split else 0)


@pytest.mark.parametrize("H,S,sinks,recent", [(8, 131072, 4, 512), (3, 20000, 0, 0), (5, 150001, 4, 64)])
def test_evict_select_prepare_on_given_scores(H, S, sinks, recent):
    """evict_select_prepare on given scores (mass-like heavy tails, ties,
    -0.0, NaN and infinities), then several budget sets on the one workspace;
    150001 positions exceed the three-launch select (nothing prepared)."""
    say(f"evict_select_prepare H={H} S={S} sinks={sinks} recent={recent}")
    g = torch.Generator().manual_seed(H * 1000 + S)
    x = torch.exp(torch.randn(H, S, generator=g) * 3.0)
    x[:, ::97] = x[:, 5:6]                     # ties
    x[0, 10:20] = float("nan")
    x[-1, 30:40] = -0.0
    x[-1, 41] = float("inf")
    x[0, 42] = float("-inf")
    scores = x.to(DEV)
    ws = fam.evict_select_prepare(scores, sinks, recent)
    for seed in range(3):
        budgets = budgets_for(seed, H, S, sinks, recent)
        idx, off = fam.evict_select_prepared(scores, budgets, sinks, recent, ws)
        ref_idx, ref_off = fam.evict_select(scores, budgets, sinks, recent)
        torch.cuda.synchronize()
        assert torch.equal(off, ref_off) and torch.equal(idx, ref_idx), f"budgets {budgets}"
    o_idx, _ = so.select(x.numpy(), budgets, sinks, recent)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
