"""GPU parity of fam_lse / fam_mass / fam_compute against the fp64 oracle.

Tolerances (from the method's stated bar): |lse_gpu - lse_ref| <= 1e-3, and
|mass_gpu - mass_ref| / mass_ref <= 2e-3 on every key with mass_ref > 0; keys
that no query can reach (j > S - 1 - W) must be exactly 0. The GPU reads bf16
(or fp16) inputs and the oracle reads the same values converted exactly to
fp64.

Sizes the oracle finishes in seconds are compared element by element (the
32k and 128k workloads against stored oracle results in
tests/test_gpu_fullsize.py), and properties that hold at any size (the W = 0
column-sum invariant, the uniform and single-sink closed forms) are checked
on every output.
"""
import math

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads
from oracle import fam_oracle as fo

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3
MASS_RTOL = 2e-3
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def check_lse(got, ref):
    err = np.abs(np.asarray(got, np.float64) - ref).max()
    assert err <= LSE_TOL, f"lse max abs err {err}"
    return err


def check_mass(got, ref, S, W):
    got = np.asarray(got, np.float64)
    if W < S:
        assert np.all(got[..., S - W:] == 0.0), "unreachable keys must be exactly 0"
    else:
        assert np.all(got == 0.0)
    pos = ref > 0
    if pos.any():
        rel = np.abs(got[pos] - ref[pos]) / np.maximum(ref[pos], np.finfo(np.float32).tiny)
        assert rel.max() <= MASS_RTOL, f"mass max rel err {rel.max()}"
        return rel.max()
    return 0.0


def rand_inputs(seed, B, Hq, Hkv, S, d, dtype, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, S, d, generator=g) * spread).to(dtype)
    k = (torch.randn(B, Hkv, S, d, generator=g) * spread).to(dtype)
    return q, k


SMALL = [
    # (seed, B, Hq, Hkv, S, d, W, dtype)
    (1, 1, 4, 1, 1, 128, 0, torch.bfloat16),
    (2, 1, 4, 2, 7, 64, 3, torch.bfloat16),
    (3, 2, 8, 2, 100, 128, 10, torch.bfloat16),
    (4, 1, 4, 4, 333, 64, 0, torch.bfloat16),
    (5, 1, 8, 1, 1000, 128, 64, torch.bfloat16),
    (6, 1, 2, 1, 257, 128, 300, torch.bfloat16),
    (7, 1, 4, 2, 640, 128, 31, torch.float16),
    (8, 1, 3, 3, 129, 64, 1, torch.bfloat16),
    (9, 1, 6, 2, 200, 128, 5, torch.bfloat16),
    (10, 1, 16, 2, 300, 64, 7, torch.bfloat16),
    (11, 1, 4, 1, 1537, 128, 513, torch.bfloat16),
    (12, 1, 2, 2, 2048, 64, 2047, torch.float16),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,d,W,dtype", SMALL)
def test_small_and_ragged_against_full_oracle(seed, B, Hq, Hkv, S, d, W, dtype):
    say(f"small seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W} {dtype}")
    q, k = rand_inputs(seed, B, Hq, Hkv, S, d, dtype, spread=1.3)
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), W)
    torch.cuda.synchronize()
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), W)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, S, W)


def test_explicit_scale_and_strided_views():
    say("explicit scale, non-contiguous head stride")
    S, d = 384, 128
    base = torch.randn(1, 8, S, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q = base[:, ::2]                       # head stride 2*S*d
    k = torch.randn(1, 2, S, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), 16, scale=0.05)
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), 16, scale=0.05)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, S, 16)


@pytest.mark.parametrize("scale", [1e-30, 1e-12, 0.5, 1.0])
def test_scales_from_the_smallest_accepted_to_sharp(scale):
    """The mass pass starts each row's accumulators at -lse / c (c = scale *
    log2 e) and forms exp2(c * acc); at tiny scales -lse / c reaches ~1e31
    and swamps every dot product, at 1.0 (11x the default at d = 128) the
    normalisers reach 87 and the masses span 23 decades (sharper scales put
    masses below what fp32 represents, which would test the number format
    rather than the kernels). Both passes against the oracle at the parity
    bar, and the per-query-head mass summed over each group against the
    group mass."""
    say(f"scale {scale}")
    q, k = rand_inputs(31, 1, 4, 2, 300, 128, torch.bfloat16, spread=1.3)
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), 5, scale=scale)
    mass_q = fam.fam_mass_per_head(q.to(DEV), k.to(DEV), lse, 5, scale=scale)
    torch.cuda.synchronize()
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), 5, scale=scale)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, 300, 5)
    grp = mass_q.view(1, 2, 2, 300).sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(grp, mass.cpu().numpy(), rtol=1e-5, atol=0)


def test_tiny_workload_full_oracle():
    wl = workloads.tiny()
    say(wl.name)
    t = wl.tensors(with_v=False)
    lse, mass = fam.fam_compute(t["q"].to(DEV), t["k"].to(DEV), wl.W)
    lse_ref, mass_ref = fo.fam(to64(t["q"]), to64(t["k"]), wl.W)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, wl.S, wl.W)


def test_qwen3_4b_layer_two_groups_full_oracle():
    wl = workloads.qwen3_4b_layer()
    say(wl.name)
    t = wl.tensors(with_v=False)
    lse, mass = fam.fam_compute(t["q"].to(DEV), t["k"].to(DEV), wl.W)
    lse, mass = lse.cpu().numpy()[0], mass.cpu().numpy()[0]
    g = wl.group
    for h in (0, wl.Hkv - 1):
        qg = to64(t["q"][0, h * g:(h + 1) * g])
        kh = to64(t["k"][0, h:h + 1])
        lse_ref, mass_ref = fo.fam(qg, kh, wl.W)
        check_lse(lse[h * g:(h + 1) * g], lse_ref)
        check_mass(mass[h:h + 1], mass_ref, wl.S, wl.W)


@pytest.mark.parametrize("S,Hq,Hkv,d", [(8192, 32, 8, 128), (131072, 32, 8, 128), (5000, 6, 2, 64),
                                        (524288, 4, 1, 128)])
def test_w0_invariant_full_size(S, Hq, Hkv, d):
    say(f"W=0 invariant S={S} Hq={Hq} Hkv={Hkv} d={d}")
    gen = torch.Generator(device=DEV).manual_seed(S)
    q = torch.randn(1, Hq, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    k = torch.randn(1, Hkv, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    _, mass = fam.fam_compute(q, k, 0)
    tot = mass.double().sum(dim=-1).cpu().numpy()[0]
    g = Hq // Hkv
    rel = np.abs(tot / (S * g) - 1.0).max()
    print(f"W=0 column total: max rel err {rel:.2e}", flush=True)
    np.testing.assert_allclose(tot, np.full(Hkv, S * g), rtol=1e-5)


def harmonic_prefix(n):
    return np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1, dtype=np.float64))])


@pytest.mark.parametrize("S,W", [(131072, 512), (32768, 256), (3000, 0), (524288, 1024)])
def test_uniform_logits_closed_form_full_size(S, W):
    say(f"uniform closed form S={S} W={W}")
    Hq, Hkv, d = 8, 2, 128
    q = torch.zeros(1, Hq, S, d, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(1, Hkv, S, d, device=DEV, generator=torch.Generator(device=DEV).manual_seed(1)).to(torch.bfloat16)
    lse, mass = fam.fam_compute(q, k, W)
    Hn = harmonic_prefix(S)
    lse_ref = np.log(np.arange(1, S + 1, dtype=np.float64))
    check_lse(lse.cpu().numpy()[0], lse_ref[None, :])
    j = np.arange(S)
    ref = np.where(j <= S - 1 - W, (Hq // Hkv) * (Hn[S] - Hn[np.minimum(j + W, S)]), 0.0)
    check_mass(mass.cpu().numpy()[0], np.broadcast_to(ref, (Hkv, S)), S, W)


def mass_parts(t):
    """Per-launch ranges of the mass pass in range mode: 64 tiles of 64 query rows each."""
    return -(-(-(-t // 64)) // 64)


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,d,W", [(51, 1, 8, 2, 65613, 128, 300), (52, 2, 4, 1, 70000, 64, 0),
                                                 (53, 1, 4, 2, 65536, 128, 4095)])
def test_range_mass_matches_even_splits_and_unsplit(seed, B, Hq, Hkv, S, d, W):
    """From 65536 keys on, with fam_mass_workspace_size bytes, every range of
    4096 query rows gets its own workgroup per key block; with room for fewer
    parts the pass splits each block's steps evenly, and without a workspace
    it runs unsplit. The three agree to fp32 rounding (the same products,
    added in another order), unreachable keys are exactly 0 in each, and at
    W = 0 every query head's mass sums to S."""
    say(f"range mass seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W}")
    per = B * Hkv * S * 4
    nr = mass_parts(S)
    assert fam.fam_mass_workspace_size(B, Hq, Hkv, S) == nr * per
    gen = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, Hq, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    lse = fam.fam_lse(q, k, knorm=fam.fam_key_norms(k))
    ranged = fam.fam_mass(q, k, lse, W)
    even = fam.fam_mass(q, k, lse, W, workspace=torch.empty((nr - 1) * per, dtype=torch.uint8, device=DEV))
    whole = fam.fam_mass(q, k, lse, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    pos = whole > 0
    assert torch.all(whole[..., S - W:] == 0) and torch.all(ranged[..., S - W:] == 0)
    for other, name in ((ranged, "ranges"), (even, "even splits")):
        assert torch.equal(other[~pos], whole[~pos]), name
        rel = ((other - whole).abs()[pos] / whole[pos]).max().item()
        assert rel <= 1e-5, f"{name}: max rel diff {rel}"
    if W == 0:
        tot = ranged.double().sum(dim=-1).cpu().numpy()
        np.testing.assert_allclose(tot, np.full((B, Hkv), S * (Hq // Hkv)), rtol=1e-5)


@pytest.mark.parametrize("dtype,strided", [(torch.float16, False), (torch.bfloat16, True)])
def test_range_mass_fp16_and_strided_views(dtype, strided):
    """Ranges of query rows on fp16 inputs, and on bf16 views whose rows sit
    in wider buffers (row stride 2d, the head dim contiguous) with the head
    and batch strides of a transposed [B, S, H, 2d] layout: equal to the
    unsplit pass to fp32 rounding, the same zeros, and the group sum of the
    per-query-head ranges equal to fam_mass."""
    B, Hq, Hkv, S, d, W = 1, 4, 2, 65600, 128, 64
    say(f"range mass {dtype} strided={strided} S={S}")
    gen = torch.Generator(device=DEV).manual_seed(77)
    if strided:
        qb = torch.randn(B, S, Hq, 2 * d, device=DEV, generator=gen).to(dtype)
        kb = torch.randn(B, S, Hkv, 2 * d, device=DEV, generator=gen).to(dtype)
        q = qb[..., :d].permute(0, 2, 1, 3)   # [B, Hq, S, d] view, row stride Hq * 2d
        k = kb[..., d:].permute(0, 2, 1, 3)
        assert not q.is_contiguous() and q.stride(3) == 1
    else:
        q = torch.randn(B, Hq, S, d, device=DEV, generator=gen).to(dtype)
        k = torch.randn(B, Hkv, S, d, device=DEV, generator=gen).to(dtype)
    lse = fam.fam_lse(q, k, knorm=fam.fam_key_norms(k))
    ranged = fam.fam_mass(q, k, lse, W)
    whole = fam.fam_mass(q, k, lse, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    pos = whole > 0
    assert torch.equal(ranged[~pos], whole[~pos])
    assert ((ranged - whole).abs()[pos] / whole[pos]).max().item() <= 1e-5
    per_head = fam.fam_mass_per_head(q, k, lse, W)
    summed = per_head.view(B, Hkv, Hq // Hkv, S).double().sum(2)
    assert torch.all(summed[~pos] == 0)
    assert ((summed - whole.double()).abs()[pos] / whole.double()[pos]).max().item() <= 1e-5


@pytest.mark.parametrize("W", [65536, 100000, 65535])
def test_range_mass_window_edges(W):
    """Ranges of query rows with a window that leaves no future query (W >= S:
    every mass is exactly 0) or one (W = S - 1: only key 0, from the last
    query, in the last range), against the unsplit pass and the oracle's
    value for the one key."""
    B, Hq, Hkv, S, d = 1, 4, 2, 65536, 128
    say(f"range mass window edge S={S} W={W}")
    gen = torch.Generator(device=DEV).manual_seed(W)
    q = torch.randn(B, Hq, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, d, device=DEV, generator=gen).to(torch.bfloat16)
    lse = fam.fam_lse(q, k, knorm=fam.fam_key_norms(k))
    ranged = fam.fam_mass(q, k, lse, W)
    whole = fam.fam_mass(q, k, lse, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    if W >= S:
        assert torch.all(ranged == 0) and torch.all(whole == 0)
        return
    assert torch.all(ranged[..., 1:] == 0) and torch.all(whole[..., 1:] == 0)
    g, scale = Hq // Hkv, 1.0 / math.sqrt(d)
    for h in range(Hkv):
        qg = to64(q[0, h * g:(h + 1) * g])
        kh = to64(k[0, h])
        lse_tail = np.stack([fo.causal_lse_rows(qg[n], kh, np.array([S - 1]), scale) for n in range(g)])
        ref = fo.future_mass_keys(qg, kh, lse_tail, S - 1, np.array([0]), W, scale)[0]
        for got in (ranged, whole):
            assert abs(got[0, h, 0].item() - ref) <= MASS_RTOL * ref


@pytest.mark.parametrize("Sq,Sk,W", [(8256, 70000, 0), (12288, 65536, 200)])
def test_range_mass_of_a_chunk(Sq, Sk, W):
    """A chunk of Sq >= 4096 queries over Sk >= 65536 cache rows runs the mass
    pass in ranges of the chunk's own rows; it agrees with the call without a
    workspace, and at W = 0 each query head's mass sums to Sq."""
    B, Hq, Hkv, d = 1, 8, 2, 128
    say(f"range mass of a chunk Sq={Sq} Sk={Sk} W={W}")
    gen = torch.Generator(device=DEV).manual_seed(Sq + Sk)
    q = torch.randn(B, Hq, Sq, d, device=DEV, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Sk, d, device=DEV, generator=gen).to(torch.bfloat16)
    assert fam.fam_compute_workspace_size(B, Hq, Hkv, Sq, Sk) >= mass_parts(Sq) * B * Hkv * Sk * 4
    lse_r, ranged = fam.fam_compute_chunk(q, k, W)
    lse_w, whole = fam.fam_compute_chunk(q, k, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    assert (lse_r - lse_w).abs().max().item() <= 1e-5
    pos = whole > 0
    assert torch.equal(ranged[~pos], whole[~pos])
    assert ((ranged - whole).abs()[pos] / whole[pos]).max().item() <= 2e-5
    if W == 0:
        tot = ranged.double().sum(dim=-1).cpu().numpy()
        np.testing.assert_allclose(tot, np.full((B, Hkv), Sq * (Hq // Hkv)), rtol=1e-5)


@pytest.mark.parametrize("S,W,a,b", [(65536, 100, 4.0, 4.0), (777, 3, 8.0, 2.0)])
def test_single_sink_closed_form(S, W, a, b):
    say(f"single sink S={S} W={W}")
    Hq, Hkv, d = 4, 1, 128
    q = torch.zeros(1, Hq, S, d, dtype=torch.bfloat16)
    q[..., 0] = a
    k = torch.zeros(1, Hkv, S, d, dtype=torch.bfloat16)
    k[0, 0, 0, 0] = b
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), W)
    c = a * b / math.sqrt(d)
    ec = math.exp(c)
    i = np.arange(S, dtype=np.float64)
    check_lse(lse.cpu().numpy()[0], np.log(ec + i)[None, :])
    inv = 1.0 / (ec + i)
    suffix = np.concatenate([np.cumsum(inv[::-1])[::-1], [0.0]])  # suffix[m] = sum_{i>=m} inv
    ref = np.zeros(S)
    ref[0] = Hq * ec * suffix[min(W, S)]
    jj = np.arange(1, S)
    ref[1:] = Hq * suffix[np.minimum(jj + W, S)]
    check_mass(mass.cpu().numpy()[0], ref[None, :], S, W)


def test_deterministic_bitwise():
    say("determinism")
    q, k = rand_inputs(21, 1, 8, 2, 4099, 128, torch.bfloat16)
    q, k = q.to(DEV), k.to(DEV)
    a = fam.fam_compute(q, k, 64)
    b = fam.fam_compute(q, k, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_separate_passes_match_compute():
    """fam_compute shifts the exponentials by a key-norm bound, fam_lse by the
    running maximum; both must meet the oracle and agree to fp32 rounding."""
    say("fam_lse + fam_mass vs fam_compute")
    q, k = rand_inputs(22, 1, 4, 1, 999, 64, torch.bfloat16)
    qd, kd = q.to(DEV), k.to(DEV)
    lse = fam.fam_lse(qd, kd)
    mass = fam.fam_mass(qd, kd, lse, 17)
    lse2, mass2 = fam.fam_compute(qd, kd, 17)
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), 17)
    for l_, m_ in ((lse, mass), (lse2, mass2)):
        check_lse(l_.cpu().numpy(), lse_ref)
        check_mass(m_.cpu().numpy(), mass_ref, 999, 17)
    assert (lse - lse2).abs().max().item() <= 1e-5
    pos = mass2 > 0
    assert ((mass - mass2).abs()[pos] / mass2[pos]).max().item() <= 1e-5


def orthogonal_big_norm_inputs(S, d, big, seed):
    """Queries and keys whose large components lie in different coordinates:
    the logits stay O(1) while |q| * |k| is huge, so the Cauchy-Schwarz row
    bound is far too high and every row's bounded sum underflows."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(1, 2, S, d, generator=g)
    k = torch.randn(1, 1, S, d, generator=g)
    q[..., 0], q[..., 1] = big, 0.0       # query rows: large along axis 0
    k[..., 0], k[..., 1] = 0.0, 0.0
    k[0, 0, 0, 1] = big                   # one key: large along axis 1
    return q.to(torch.bfloat16), k.to(torch.bfloat16)


@pytest.mark.parametrize("S,big", [(300, 200.0), (2049, 64.0)])
def test_loose_bound_falls_back_to_running_max(S, big):
    say(f"loose key-norm bound S={S} big={big}")
    q, k = orthogonal_big_norm_inputs(S, 128, big, seed=S)
    W = 9
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), W)
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), W)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, S, W)


def test_moderately_loose_bound_without_fallback():
    """One key six times longer than the rest: the bound exceeds most rows'
    maxima by tens of log2 units but the sums stay far above the fallback
    threshold."""
    say("moderately loose bound")
    q, k = rand_inputs(23, 1, 8, 2, 1500, 128, torch.bfloat16)
    k[0, :, 7] *= 6
    lse, mass = fam.fam_compute(q.to(DEV), k.to(DEV), 20)
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), 20)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, 1500, 20)


@pytest.mark.parametrize("B,H,S,d,dtype", [(1, 8, 131072, 128, torch.bfloat16), (2, 3, 100, 128, torch.bfloat16),
                                           (1, 2, 5, 64, torch.float16), (1, 1, 4097, 64, torch.bfloat16)])
def test_key_norms_against_float64(B, H, S, d, dtype):
    say(f"key norms B={B} H={H} S={S} d={d} {dtype}")
    g = torch.Generator().manual_seed(S)
    k = (torch.randn(B, H, S, d, generator=g) * 3).to(dtype)
    kn = fam.fam_key_norms(k.to(DEV)).cpu().double()
    P = fam.fam_key_norm_parts(S)
    chunk = -(-S // P)
    sq = (k.double() ** 2).sum(-1)
    padded = torch.zeros(B, H, P * chunk, dtype=torch.float64)
    padded[..., :S] = sq
    ref = padded.view(B, H, P, chunk).max(-1).values
    assert kn.shape == (B, H, P)
    assert ((kn - ref).abs() / ref.clamp_min(1e-30)).max().item() <= 1e-5


@pytest.mark.parametrize("seed,S,d,W", [(24, 777, 128, 5), (25, 2050, 64, 300)])
def test_lse_bounded_form_against_oracle(seed, S, d, W):
    say(f"fam_lse with key norms S={S} d={d}")
    q, k = rand_inputs(seed, 1, 8, 2, S, d, torch.bfloat16, spread=1.3)
    qd, kd = q.to(DEV), k.to(DEV)
    kn = fam.fam_key_norms(kd)
    lse = fam.fam_lse(qd, kd, knorm=kn)
    mass = fam.fam_mass(qd, kd, lse, W)
    lse_ref, mass_ref = fo.fam(to64(q), to64(k), W)
    check_lse(lse.cpu().numpy(), lse_ref)
    check_mass(mass.cpu().numpy(), mass_ref, S, W)


def test_lse_bounded_form_fallback():
    say("fam_lse with key norms, loose bound")
    q, k = orthogonal_big_norm_inputs(640, 128, 100.0, seed=7)
    qd, kd = q.to(DEV), k.to(DEV)
    lse = fam.fam_lse(qd, kd, knorm=fam.fam_key_norms(kd))
    check_lse(lse.cpu().numpy()[0], fo.causal_lse(to64(q)[0], to64(k)[0]))


@pytest.mark.parametrize("seed,Hq,Hkv,S,d,W", [(41, 8, 2, 3000, 128, 100), (42, 4, 4, 700, 64, 0),
                                             (43, 32, 8, 8192, 128, 128)])
def test_split_mass_matches_unsplit_and_oracle(seed, Hq, Hkv, S, d, W):
    """Short sequences split each key block's queries over several workgroups
    (workspace of fam_mass_workspace_size bytes); without a workspace the pass
    runs unsplit. Both meet the oracle and agree to fp32 rounding."""
    say(f"split mass Hq={Hq} Hkv={Hkv} S={S} W={W}")
    assert fam.fam_mass_workspace_size(1, Hq, Hkv, S) > 0
    q, k = rand_inputs(seed, 1, Hq, Hkv, S, d, torch.bfloat16)
    qd, kd = q.to(DEV), k.to(DEV)
    lse = fam.fam_lse(qd, kd, knorm=fam.fam_key_norms(kd))
    split = fam.fam_mass(qd, kd, lse, W)
    whole = fam.fam_mass(qd, kd, lse, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    pos = whole > 0
    assert torch.equal(split[~pos], whole[~pos])
    assert ((split - whole).abs()[pos] / whole[pos]).max().item() <= 1e-5
    if S <= 3000:
        lse_ref, mass_ref = fo.fam(to64(q), to64(k), W)
        check_mass(split.cpu().numpy(), mass_ref, S, W)
        check_mass(whole.cpu().numpy(), mass_ref, S, W)
