"""GPU parity of the KVpop target row: per-query-head mass and the epilogue.

fam_mass_per_head is compared with the fp64 oracle's per-query-head mass
(same tolerance as the group mass: 2e-3 relative, exact zeros for keys no
query can reach) and, at every size, with fam_mass (the group sum). The
epilogue fam_kvpop_target is compared with oracle.kvpop_target on the
oracle's own per-head mass: the GPU target is log(mass / N), so the mass
tolerance becomes an absolute 2e-3 on the log (plus fp32 rounding), and keys
whose target is -inf must be -inf. The page's worked example is fed straight
into the GPU epilogue.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads
from oracle import fam_oracle as fo
from oracle import kvpop_target as kt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MASS_RTOL = 2e-3
TARGET_ATOL = 2.5e-3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def to64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def check_mass(got, ref, S, W):
    got = np.asarray(got, np.float64)
    if W < S:
        assert np.all(got[..., S - W:] == 0.0)
    else:
        assert np.all(got == 0.0)
    pos = ref > 0
    if pos.any():
        rel = np.abs(got[pos] - ref[pos]) / np.maximum(ref[pos], np.finfo(np.float32).tiny)
        assert rel.max() <= MASS_RTOL, f"mass max rel err {rel.max()}"


def check_target(got, ref):
    got = np.asarray(got, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "-inf positions differ"
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        assert err <= TARGET_ATOL, f"target max abs err {err}"


def rand(seed, B, Hq, Hkv, S, d, dtype=torch.bfloat16, spread=1.3):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, S, d, generator=g) * spread).to(dtype)
    k = (torch.randn(B, Hkv, S, d, generator=g) * spread).to(dtype)
    return q, k


CASES = [
    # (seed, B, Hq, Hkv, S, d, W, dtype)
    (31, 1, 4, 1, 1, 128, 0, torch.bfloat16),
    (32, 1, 4, 2, 300, 128, 7, torch.bfloat16),
    (33, 2, 6, 2, 257, 64, 0, torch.float16),
    (34, 1, 8, 2, 1100, 128, 64, torch.bfloat16),
    (35, 1, 3, 3, 200, 64, 250, torch.bfloat16),
    (36, 1, 16, 2, 600, 128, 31, torch.bfloat16),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,d,W,dtype", CASES)
def test_mass_per_head_and_target_against_oracle(seed, B, Hq, Hkv, S, d, W, dtype):
    say(f"per-head mass + target seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W} {dtype}")
    q, k = rand(seed, B, Hq, Hkv, S, d, dtype)
    qd, kd = q.to(DEV), k.to(DEV)
    lse, mass = fam.fam_compute(qd, kd, W)
    mass_q = fam.fam_mass_per_head(qd, kd, lse, W)
    torch.cuda.synchronize()
    g = Hq // Hkv
    # the group sum of the per-head masses is the group mass
    summed = mass_q.view(B, Hkv, g, S).double().sum(2)
    pos = mass.double() > 0
    assert torch.all(summed[~pos] == 0)
    if pos.any():
        assert ((summed - mass.double()).abs()[pos] / mass.double()[pos]).max().item() <= 1e-5
    mq = mass_q.cpu().numpy()
    for b in range(B):
        lse_ref = fo.causal_lse(to64(q[b]), to64(k[b]))
        _, per_q = fo.future_mass(to64(q[b]), to64(k[b]), lse_ref, W, per_query_head=True)
        check_mass(mq[b], per_q, S, W)
        for agg in ("max", "mean"):
            for eps in (0.0, 1e-6):
                tgt = fam.fam_kvpop_target(mass_q, Hkv, W, eps=eps, aggregate=agg).cpu().numpy()
                for h in range(Hkv):
                    ref = kt.target(per_q[h * g:(h + 1) * g], W, eps=eps, aggregate=agg)
                    check_target(tgt[b, h], ref)


def test_target_worked_example_on_gpu():
    """KVpop "Defining Future Attention Utility": S = 6, key t = 2, window
    w = 2, two query heads with future probabilities (0.30, 0.20) and
    (0.10, 0.10): N_t = 2, means 0.25 and 0.10, logs -1.386 and -2.303, and
    the max-aggregated target -1.386."""
    with open(os.path.join(GOLDEN, "kvpop_worked_example.json")) as f:
        ex = json.load(f)
    say("KVpop worked example through fam_kvpop_target")
    S, t, w = ex["S"], ex["t"], ex["w"]
    per_head = [sum(p) for p in ex["future_probabilities_per_query_head"]]
    mass_q = torch.zeros(1, len(per_head), S, dtype=torch.float32)
    for n, m in enumerate(per_head):
        mass_q[0, n, t] = m
    got = fam.fam_kvpop_target(mass_q.to(DEV), 1, w, eps=0.0, aggregate="max").cpu()
    dec = ex["printed_decimals"]
    assert round(float(got[0, 0, t]), dec) == ex["target_max_aggregate"]
    assert float(got[0, 0, t]) == pytest.approx(math.log(0.25), abs=1e-6)
    mean = fam.fam_kvpop_target(mass_q.to(DEV), 1, w, eps=0.0, aggregate="mean").cpu()
    assert float(mean[0, 0, t]) == pytest.approx(math.log(0.175), abs=1e-6)
    # keys with zero mass and eps = 0: log 0
    assert torch.isneginf(got[0, 0, :t]).all() and torch.isneginf(got[0, 0, t + 1:]).all()


@pytest.mark.parametrize("Hq,Hkv,S,offset", [(3, 1, 400, 0), (5, 1, 401, 0), (16, 1, 64, 0), (8, 2, 4096, 0),
                                              (4, 2, 1000, 1), (2, 1, 8, 0), (6, 3, 12, 0)])
def test_target_vector_and_scalar_paths(Hq, Hkv, S, offset):
    """Both aggregates against the oracle's epilogue on random masses: four
    keys per thread (S % 4 == 0, 16-byte aligned rows) and one key per thread
    (S odd, or rows shifted by one float), for group sizes with a
    compile-time loop (1, 2, 4, 8) and without one (3, 5, 16)."""
    say(f"kvpop target paths Hq={Hq} Hkv={Hkv} S={S} offset={offset}")
    g = torch.Generator().manual_seed(Hq * 1000 + S)
    flat = torch.rand(Hq * S + offset, generator=g) ** 4   # masses over many orders of magnitude
    flat[::7] = 0.0                                          # zero masses: log(eps) or -inf
    mass_q = flat.to(DEV)[offset:].view(1, Hq, S)
    W, gq = 5, Hq // Hkv
    for agg in ("max", "mean"):
        for eps in (0.0, 1e-6):
            got = fam.fam_kvpop_target(mass_q, Hkv, W, eps=eps, aggregate=agg).cpu().numpy()[0]
            mq = mass_q[0].double().cpu().numpy()
            for h in range(Hkv):
                check_target(got[h], kt.target(mq[h * gq:(h + 1) * gq], W, eps=eps, aggregate=agg))


def test_counts_floor_at_one_on_gpu():
    """N_j = max(1, S - (j + W)): keys in and past the window divide by 1."""
    say("count floor")
    S, W = 50, 45
    mass_q = torch.rand(1, 2, S, generator=torch.Generator().manual_seed(3)) + 0.1
    got = fam.fam_kvpop_target(mass_q.to(DEV), 1, W, aggregate="max").cpu().numpy()[0, 0]
    ref = kt.target(mass_q[0].double().numpy(), W, aggregate="max")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6)


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,d,W", [(61, 1, 8, 2, 65613, 128, 300), (62, 2, 4, 1, 70000, 64, 0)])
def test_per_head_ranges_match_unsplit(seed, B, Hq, Hkv, S, d, W):
    """From 65536 keys on, with fam_mass_per_head_workspace_size bytes, each
    range of 4096 query rows gets its own workgroup per key block and the
    parts are added per query head. Against the unsplit pass (an empty
    workspace): equal to fp32 rounding, exactly 0 on the same keys; the
    group sum equals fam_mass; at W = 0 every query head's mass sums to S."""
    say(f"per-head ranges seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W}")
    nr = -(-(-(-S // 64)) // 64)
    assert fam.fam_mass_per_head_workspace_size(B, Hq, Hkv, S) == nr * B * Hq * S * 4
    gen = torch.Generator(device=DEV).manual_seed(seed)
    qd = torch.randn(B, Hq, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    kd = torch.randn(B, Hkv, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    lse = fam.fam_lse(qd, kd, knorm=fam.fam_key_norms(kd))
    ranged = fam.fam_mass_per_head(qd, kd, lse, W)
    whole = fam.fam_mass_per_head(qd, kd, lse, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    # a workspace one slice short of the ranges runs the unsplit pass
    short = fam.fam_mass_per_head(qd, kd, lse, W,
                                  workspace=torch.empty((nr - 1) * B * Hq * S * 4, dtype=torch.uint8, device=DEV))
    assert torch.equal(short, whole)
    pos = whole > 0
    assert torch.all(whole[..., S - W:] == 0)
    assert torch.equal(ranged[~pos], whole[~pos])
    assert ((ranged - whole).abs()[pos] / whole[pos]).max().item() <= 1e-5
    mass = fam.fam_mass(qd, kd, lse, W)
    summed = ranged.view(B, Hkv, Hq // Hkv, S).double().sum(2)
    gpos = mass.double() > 0
    assert torch.all(summed[~gpos] == 0)
    assert ((summed - mass.double()).abs()[gpos] / mass.double()[gpos]).max().item() <= 1e-5
    if W == 0:
        np.testing.assert_allclose(ranged.double().sum(dim=-1).cpu().numpy(), np.full((B, Hq), S), rtol=1e-4)


def test_llama_128k_per_head_tail_keys():
    """At full size: every per-head mass sums to the group mass, and the
    per-head masses of the keys whose future queries lie in the last rows
    match the oracle."""
    wl = workloads.llama31_8b_128k()
    say(wl.name)
    t = wl.tensors(with_v=False)
    qd, kd = t["q"].to(DEV), t["k"].to(DEV)
    lse, mass = fam.fam_compute(qd, kd, wl.W)
    mass_q = fam.fam_mass_per_head(qd, kd, lse, wl.W)
    g, S, W = wl.group, wl.S, wl.W
    summed = mass_q.view(1, wl.Hkv, g, S).double().sum(2)
    pos = mass.double() > 0
    assert ((summed - mass.double()).abs()[pos] / mass.double()[pos]).max().item() <= 1e-5
    group, tail = 6, 512
    qg = to64(t["q"][0, group * g:(group + 1) * g])
    kh = to64(t["k"][0, group])
    scale = 1.0 / math.sqrt(wl.d)
    tail_start = S - tail
    keys = np.arange(tail_start - W, S)
    mq = mass_q.cpu().numpy()[0]
    for n in range(g):
        lse_tail = fo.causal_lse_rows(qg[n], kh, np.arange(tail_start, S), scale)[None]
        ref = fo.future_mass_keys(qg[n:n + 1], kh, lse_tail, tail_start, keys, W, scale)
        full = np.zeros(S)
        full[keys] = ref
        got = np.zeros(S)
        got[keys] = mq[group * g + n, keys]
        check_mass(got, full, S, W)
