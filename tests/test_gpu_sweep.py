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
fp32 rounding), then the chunk mode on the same inputs: the last Sq rows as
the chunk's queries over all S keys, against the oracle's chunk functions.
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam
from oracle import chunked as ch
from oracle import fam_oracle as fo

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 1e-3
MASS_RTOL = 2e-3


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
        lse_cref = ch.chunk_lse(qn[b, :, S - Sq:], kn[b], pos, S - Sq)
        mass_cref = ch.chunk_mass(qn[b, :, S - Sq:], kn[b], pos, lse_cref, S - Sq, W)
        check_lse(to64(lse_c[b]), lse_cref)
        check_mass(to64(mass_c[b]), mass_cref)
    grp = mass_q.view(B, Hkv, Hq // Hkv, S).double().sum(2)
    np.testing.assert_allclose(grp.cpu().numpy(), to64(mass), rtol=1e-5, atol=0)
