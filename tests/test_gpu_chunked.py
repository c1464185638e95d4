"""GPU parity of the chunked prefill-compress path against the fp64 oracle.

fam_compute_chunk is compared with oracle.chunked (which works on
positions, not rows) at the bar of the dense passes: |lse - ref| <= 1e-3 and
2e-3 relative on every mass with ref > 0, exact zeros where no chunk query
counts a key. Caches with position gaps (as after evictions, with the window
rows just before the chunk) pin the reading of rows as positions. With
Sq = Sk the call must equal fam_compute bit for bit.

kv_append and kv_compact_inplace are bit copies: compared bitwise with
numpy gathers, positions included.

The loop (ChunkedCache) is checked step by step: at every chunk the GPU's
normalisers and masses against the oracle evaluated on the GPU's own cache
state, the kept rows bit-exact against the oracle's selection fed the GPU's
mass, and the compacted cache bitwise against a gather of the previous
cache. The uniform-logit closed form (the earliest positions and the window
are kept) is checked end to end, and at the 128k Llama-like layer the final
chunk's normalisers and tail-key masses are sampled against the oracle.
"""
import math

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads
from oracle import chunked as ch

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
    zero = ref == 0
    assert np.all(got[zero] == 0.0), "keys no chunk query counts must be exactly 0"
    pos = ref > 0
    if pos.any():
        rel = np.abs(got[pos] - ref[pos]) / np.maximum(ref[pos], np.finfo(np.float32).tiny)
        assert rel.max() <= MASS_RTOL, f"mass max rel err {rel.max()}"


def gap_positions(rng, Sk, Sq, W, sinks=4):
    """Ascending positions of Sk cache rows whose last Sq rows are a chunk and
    whose W rows before it are the positions just before the chunk."""
    n_old = Sk - Sq
    n_win = min(W, n_old)
    n_mid = n_old - n_win
    n_sink = min(sinks, n_mid)
    p0 = n_old + 3 * n_mid + 7                     # leaves room for gaps
    mid = np.sort(rng.choice(np.arange(n_sink, p0 - n_win), size=n_mid - n_sink, replace=False))
    pos = np.concatenate([np.arange(n_sink), mid, np.arange(p0 - n_win, p0), np.arange(p0, p0 + Sq)])
    return pos.astype(np.int64), p0


CASES = [
    # (seed, B, Hq, Hkv, Sq, Sk, d, W, dtype, gaps)
    (1, 1, 4, 2, 64, 300, 128, 16, torch.bfloat16, False),
    (2, 1, 4, 1, 1, 513, 128, 0, torch.bfloat16, False),
    (3, 2, 8, 2, 257, 1000, 128, 64, torch.bfloat16, True),
    (4, 1, 2, 2, 100, 100, 64, 7, torch.float16, False),
    (5, 1, 6, 2, 33, 64, 64, 200, torch.bfloat16, False),
    (6, 1, 4, 4, 130, 700, 64, 0, torch.bfloat16, True),
    (7, 1, 16, 2, 96, 1200, 128, 40, torch.float16, True),
    (8, 1, 4, 1, 500, 501, 128, 499, torch.bfloat16, False),
    # enough key tiles for the first pass to split every row's key range
    (9, 1, 8, 2, 512, 4096, 128, 64, torch.bfloat16, True),
    (10, 1, 4, 1, 200, 2500, 64, 30, torch.float16, True),
]


@pytest.mark.parametrize("seed,B,Hq,Hkv,Sq,Sk,d,W,dtype,gaps", CASES)
def test_compute_chunk_against_oracle(seed, B, Hq, Hkv, Sq, Sk, d, W, dtype, gaps):
    say(f"fam_compute_chunk seed={seed} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} d={d} W={W} "
        f"{dtype} gaps={gaps}")
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, Sq, d, generator=g) * 1.2).to(dtype)
    k = (torch.randn(B, Hkv, Sk, d, generator=g) * 1.2).to(dtype)
    lse, mass = fam.fam_compute_chunk(q.to(DEV), k.to(DEV), W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for b in range(B):
        if gaps:
            pos, p0 = gap_positions(rng, Sk, Sq, W)
        else:
            pos, p0 = np.arange(Sk, dtype=np.int64), Sk - Sq
        P = np.tile(pos, (Hkv, 1))
        lse_ref = ch.chunk_lse(to64(q[b]), to64(k[b]), P, p0)
        mass_ref = ch.chunk_mass(to64(q[b]), to64(k[b]), P, lse_ref, p0, W)
        check_lse(to64(lse[b]), lse_ref)
        check_mass(to64(mass[b]), mass_ref)


@pytest.mark.parametrize("S,W", [(300, 16), (1, 0), (1024, 1024)])
def test_compute_chunk_full_square_equals_fam_compute(S, W):
    say(f"fam_compute_chunk Sq = Sk = {S}, W={W}")
    g = torch.Generator().manual_seed(S)
    q = torch.randn(1, 8, S, 128, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(1, 2, S, 128, generator=g).to(torch.bfloat16).to(DEV)
    l1, m1 = fam.fam_compute(q, k, W)
    l2, m2 = fam.fam_compute_chunk(q, k, W)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(m1, m2)


@pytest.mark.parametrize("Sq,Sk,loose", [(512, 4096, False), (700, 3000, True), (4096, 20480, False)])
def test_compute_chunk_split_matches_unsplit(Sq, Sk, loose):
    """With a workspace of fam_compute_workspace_size bytes the first pass
    splits every row's key range over several workgroups (and the mass pass
    its queries); with an empty one neither pass splits. Both agree to fp32
    rounding and meet the oracle. With `loose`, the query rows of the second
    half are long and orthogonal to one very long key, so their Cauchy-Schwarz
    bound is far too high: their workgroups repeat the sweep with the running
    maximum while the others keep the added partial sums."""
    say(f"fam_compute_chunk split vs unsplit Sq={Sq} Sk={Sk} loose={loose}")
    Hq, Hkv, W, d = (32, 8, 512, 128) if Sk > 10000 else (8, 2, 40, 128)
    g = torch.Generator().manual_seed(Sq + Sk)
    q = torch.randn(1, Hq, Sq, d, generator=g)
    k = torch.randn(1, Hkv, Sk, d, generator=g)
    if loose:
        q[0, :, Sq // 2:, 0], q[0, :, Sq // 2:, 1] = 40.0, 0.0
        k[0, :, :, 0], k[0, :, :, 1] = 0.0, 0.0
        k[0, :, 3, 1] = 40.0
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    qd, kd = q.to(DEV), k.to(DEV)
    assert fam.fam_compute_workspace_size(1, Hq, Hkv, Sq, Sk) > 0
    l1, m1 = fam.fam_compute_chunk(qd, kd, W)
    l0, m0 = fam.fam_compute_chunk(qd, kd, W, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert (l1 - l0).abs().max().item() <= 1e-5
    pos = m0 > 0
    assert torch.equal(m1[~pos], m0[~pos])
    assert ((m1 - m0).abs()[pos] / m0[pos]).max().item() <= 1e-5
    P = np.tile(np.arange(Sk, dtype=np.int64), (Hkv, 1))
    if Sk <= 5000:
        lse_ref = ch.chunk_lse(to64(q[0]), to64(k[0]), P, Sk - Sq)
        check_lse(to64(l1[0]), lse_ref)
        check_mass(to64(m1[0]), ch.chunk_mass(to64(q[0]), to64(k[0]), P, lse_ref, Sk - Sq, W))
    else:   # sampled rows of two query heads against the oracle
        kk = to64(k[0])
        for qh in (0, Hq - 1):
            h = qh // (Hq // Hkv)
            for r in (0, 1, 63, 64, 1000, 2047, 2048, 4000, Sq - 1):
                ref = ch.chunk_lse(to64(q[0, qh:qh + 1, r:r + 1]), kk[h:h + 1], P[:1], Sk - Sq + r)
                check_lse(to64(l1[0, qh, r:r + 1]), ref[0])


def sorted_subset(rng, S, n, keep_prefix=0):
    rest = np.sort(rng.choice(np.arange(keep_prefix, S), size=n - keep_prefix, replace=False))
    return np.concatenate([np.arange(keep_prefix), rest]).astype(np.int32)


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16), (256, torch.bfloat16)])
def test_append_and_compact_inplace_bitwise(d, dtype):
    say(f"kv_append + kv_compact_inplace d={d} {dtype}")
    H, cap = 5, 3000
    g = torch.Generator().manual_seed(d)
    k_cache = torch.randn(H, cap, d, generator=g).to(dtype).to(DEV)
    v_cache = torch.randn(H, cap, d, generator=g).to(dtype).to(DEV)
    pos = torch.full((H, cap), -1, dtype=torch.int32, device=DEV)
    n0, n1 = 1700, 900
    first_k = torch.randn(H, n0, d, generator=g).to(dtype).to(DEV)
    first_v = torch.randn(H, n0, d, generator=g).to(dtype).to(DEV)
    src_k = torch.randn(H, n1, d, generator=g).to(dtype).to(DEV)
    src_v = torch.randn(H, n1, d, generator=g).to(dtype).to(DEV)
    fam.kv_append(first_k, first_v, k_cache, v_cache, 0, pos, 0)
    fam.kv_append(src_k, src_v, k_cache, v_cache, n0, pos, 5000)
    torch.cuda.synchronize()
    n = n0 + n1
    kc, vc, pc = k_cache.cpu(), v_cache.cpu(), pos.cpu()
    assert torch.equal(kc[:, :n0], first_k.cpu()) and torch.equal(vc[:, :n0], first_v.cpu())
    assert torch.equal(kc[:, n0:n], src_k.cpu()) and torch.equal(vc[:, n0:n], src_v.cpu())
    assert torch.equal(pc[:, :n0], torch.arange(n0, dtype=torch.int32).expand(H, n0))
    assert torch.equal(pc[:, n0:n], torch.arange(5000, 5000 + n1, dtype=torch.int32).expand(H, n1))
    rng = np.random.default_rng(d)
    keeps = [sorted_subset(rng, n, 1200, keep_prefix=300),   # identity prefix, then moves
             np.arange(n, dtype=np.int32),                    # everything: no row moves
             np.zeros(0, dtype=np.int32),                     # nothing kept
             sorted_subset(rng, n, 2599),                     # all but one
             sorted_subset(rng, n, 17)]                       # a few far rows
    idx = torch.from_numpy(np.concatenate(keeps)).to(DEV)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum([x.size for x in keeps])]), dtype=torch.int64,
                           device=DEV)
    # the region is the first n rows; rows past it must stay untouched
    fam.kv_compact_inplace(k_cache[:, :n], v_cache[:, :n], idx, offsets, pos[:, :n])
    torch.cuda.synchronize()
    k2, v2, p2 = k_cache.cpu(), v_cache.cpu(), pos.cpu()
    for h, keep in enumerate(keeps):
        rows = torch.from_numpy(keep.astype(np.int64))
        m = keep.size
        assert torch.equal(k2[h, :m].view(torch.int16), kc[h, rows].view(torch.int16))
        assert torch.equal(v2[h, :m].view(torch.int16), vc[h, rows].view(torch.int16))
        assert torch.equal(p2[h, :m], pc[h, rows])
        assert torch.equal(k2[h, n:], kc[h, n:]) and torch.equal(p2[h, n:], pc[h, n:])


def test_compact_inplace_matches_out_of_place_compact():
    say("kv_compact_inplace vs kv_compact on evict_select output")
    H, S, d = 8, 5000, 128
    g = torch.Generator().manual_seed(5)
    k = torch.randn(H, S, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(H, S, d, generator=g).to(torch.bfloat16).to(DEV)
    scores = torch.rand(H, S, generator=g).to(DEV)
    budgets = [100, 4000, 5000, 0, 2500, 700, 4999, 1]
    idx, offsets = fam.evict_select(scores, budgets, 4, 64)
    k_new, v_new = fam.kv_compact(k, v, idx, offsets)
    fam.kv_compact_inplace(k, v, idx, offsets)
    torch.cuda.synchronize()
    off = offsets.cpu().tolist()
    for h in range(H):
        m = off[h + 1] - off[h]
        assert torch.equal(k[h, :m], k_new[off[h]:off[h + 1]])
        assert torch.equal(v[h, :m], v_new[off[h]:off[h + 1]])


def inplace_bitwise(H, S, d, keeps, seed, workspace=None):
    """kv_compact_inplace of keeps[h] (ascending rows of head h) against a
    numpy gather of the original cache, K, V and positions bit for bit."""
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(H, S, d, generator=g).to(torch.bfloat16)
    v = torch.randn(H, S, d, generator=g).to(torch.bfloat16)
    pos = torch.randint(0, 1 << 30, (H, S), generator=g, dtype=torch.int32)
    kd, vd, pd = k.to(DEV), v.to(DEV), pos.to(DEV)
    idx = torch.from_numpy(np.concatenate(keeps).astype(np.int32)).to(DEV)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum([x.size for x in keeps])]), dtype=torch.int64,
                           device=DEV)
    fam.kv_compact_inplace(kd, vd, idx, offsets, pd, workspace=workspace)
    torch.cuda.synchronize()
    k2, v2, p2 = kd.cpu(), vd.cpu(), pd.cpu()
    for h, keep in enumerate(keeps):
        rows = torch.from_numpy(keep.astype(np.int64))
        m = keep.size
        assert torch.equal(k2[h, :m].view(torch.int16), k[h, rows].view(torch.int16)), f"head {h}"
        assert torch.equal(v2[h, :m].view(torch.int16), v[h, rows].view(torch.int16)), f"head {h}"
        assert torch.equal(p2[h, :m], pos[h, rows]), f"head {h}"
        # only rows below m are written
        assert torch.equal(k2[h, m:].view(torch.int16), k[h, m:].view(torch.int16)), f"head {h}"
        assert torch.equal(p2[h, m:], pos[h, m:]), f"head {h}"


def test_compact_inplace_chunked_loop_shape_twice():
    """The 128k loop's compression (8 heads of 20480 rows keeping 16384, sinks
    and window forced): every chunk of 256 rows waits for up to 17 earlier
    ones. Two calls on one workspace, the second with fewer rows, check that
    each call clears its tickets and flags."""
    say("kv_compact_inplace 8 x 20480 -> 16384, twice on one workspace")
    H, S, keep = 8, 20480, 16384
    rng = np.random.default_rng(11)
    ws = torch.empty(fam.kv_compact_inplace_workspace_size(H * keep), dtype=torch.uint8, device=DEV)
    keeps = [np.concatenate([np.arange(4), np.sort(rng.choice(np.arange(4, S - 512), keep - 516, replace=False)),
                             np.arange(S - 512, S)]) for _ in range(H)]
    inplace_bitwise(H, S, 128, keeps, seed=1, workspace=ws)
    keeps = [sorted_subset(rng, S, int(rng.integers(0, 9000))) for _ in range(H)]
    inplace_bitwise(H, S, 128, keeps, seed=2, workspace=ws)


def test_compact_inplace_long_shift():
    """A head whose kept rows all lie 20000 rows further on: each chunk waits
    for about 80 earlier chunks (more than one batch of 64 flag polls)."""
    say("kv_compact_inplace shift of 20000 rows")
    H, S = 2, 40960
    rng = np.random.default_rng(12)
    keeps = [np.concatenate([np.arange(4), np.arange(20004, S)]), sorted_subset(rng, S, 30000)]
    inplace_bitwise(H, S, 128, keeps, seed=3)


@pytest.mark.parametrize("H,S,d", [(600, 300, 64), (40, 700, 256)])
def test_compact_inplace_many_small_heads(H, S, d):
    """Chunks that span many heads (offsets beyond the 512 kept in LDS for
    H = 600), empty heads, whole heads kept and heads keeping one row."""
    say(f"kv_compact_inplace H={H} S={S} d={d}")
    rng = np.random.default_rng(H)
    keeps = []
    for h in range(H):
        kind = h % 4
        n = {0: 0, 1: S, 2: 1, 3: int(rng.integers(1, S))}[kind]
        keeps.append(np.arange(S) if n == S else sorted_subset(rng, S, n))
    inplace_bitwise(H, S, d, keeps, seed=4)


def run_loop_checked(q, k, v, chunk, budget, sinks, W):
    """Drive ChunkedCache chunk by chunk, checking every step."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    cache = fam.ChunkedCache(B, Hq, Hkv, d, chunk, budget, sinks, W, k.dtype, DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    steps = 0
    for p0 in range(0, S, chunk):
        p1 = min(S, p0 + chunk)
        cache.append(kd[:, :, p0:p1], vd[:, :, p0:p1])
        lse, mass = cache.score(qd[:, :, p0:p1])
        torch.cuda.synchronize()
        n = cache.n
        krows = cache.k[:, :n].cpu()
        vrows = cache.v[:, :n].cpu()
        pos = cache.pos[:, :n].cpu().numpy().astype(np.int64)
        for b in range(B):
            hs = slice(b * Hkv, (b + 1) * Hkv)
            kb = krows[hs].to(torch.float64).numpy()
            lse_ref = ch.chunk_lse(to64(q[b, :, p0:p1]), kb, pos[hs], p0)
            mass_ref = ch.chunk_mass(to64(q[b, :, p0:p1]), kb, pos[hs], lse_ref, p0, W)
            check_lse(to64(lse[b]), lse_ref)
            check_mass(to64(mass[b]), mass_ref)
        idx, offsets = cache.compress()
        torch.cuda.synchronize()
        if idx is None:
            assert n <= budget
            continue
        steps += 1
        m = mass.view(B * Hkv, n).cpu().numpy().astype(np.float64)
        idx_h = idx.cpu().numpy().reshape(B * Hkv, -1)
        for h in range(B * Hkv):
            want = ch.compress_rows(m[h], pos[h], budget, sinks, W, p1)
            np.testing.assert_array_equal(idx_h[h], want)
            rows = torch.from_numpy(want)
            assert torch.equal(cache.k[h, :want.size].cpu().view(torch.int16), krows[h, rows].view(torch.int16))
            assert torch.equal(cache.v[h, :want.size].cpu().view(torch.int16), vrows[h, rows].view(torch.int16))
            np.testing.assert_array_equal(cache.pos[h, :want.size].cpu().numpy(), pos[h][want])
        assert cache.n == idx_h.shape[1]
    return cache, steps


@pytest.mark.parametrize("seed,B,Hq,Hkv,S,d,chunk,budget,sinks,W,dtype", [
    (1, 1, 4, 2, 1500, 128, 256, 400, 4, 64, torch.bfloat16),
    (2, 2, 8, 2, 900, 64, 128, 300, 4, 32, torch.float16),
    (3, 1, 4, 1, 700, 128, 100, 150, 2, 120, torch.bfloat16),   # chunk shorter than the window
])
def test_loop_step_by_step_against_oracle(seed, B, Hq, Hkv, S, d, chunk, budget, sinks, W, dtype):
    say(f"ChunkedCache seed={seed} B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} chunk={chunk} budget={budget} "
        f"sinks={sinks} W={W}")
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, S, d, generator=g) * 1.3).to(dtype)
    k = (torch.randn(B, Hkv, S, d, generator=g) * 1.3).to(dtype)
    v = torch.randn(B, Hkv, S, d, generator=g).to(dtype)
    _, steps = run_loop_checked(q, k, v, chunk, budget, sinks, W)
    assert steps >= 2


def test_loop_uniform_logits_keep_the_earliest_and_the_window():
    say("prefill_compress with q = 0")
    B, Hq, Hkv, S, d, chunk, budget, sinks, W = 1, 8, 2, 3000, 128, 512, 1000, 4, 128
    g = torch.Generator().manual_seed(9)
    q = torch.zeros(B, Hq, S, d, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(B, Hkv, S, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, Hkv, S, d, generator=g).to(torch.bfloat16).to(DEV)
    cache = fam.prefill_compress(q, k, v, chunk, budget, sinks, W)
    torch.cuda.synchronize()
    want = np.concatenate([np.arange(budget - W), np.arange(S - W, S)])
    assert cache.n == want.size
    rows = torch.from_numpy(want)
    for h in range(Hkv):
        np.testing.assert_array_equal(cache.pos[h, :cache.n].cpu().numpy(), want)
        assert torch.equal(cache.k[h, :cache.n].cpu(), k[0, h].cpu()[rows])
        assert torch.equal(cache.v[h, :cache.n].cpu(), v[0, h].cpu()[rows])


def test_llama_128k_chunked_final_chunk_sampled():
    """128k Llama-like layer, chunks of 4096, budget 16384 per head: cache
    invariants, and the final chunk's sampled normalisers and the masses of
    the keys counted only by its last 64 queries, against the oracle."""
    wl = workloads.llama31_8b_128k()
    say(f"{wl.name} chunked prefill-compress")
    t = wl.tensors(with_v=True)
    qd, kd, vd = t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV)
    chunk, budget, sinks, W = 4096, 16384, wl.sinks, wl.W
    B, Hq, S, d = qd.shape
    Hkv = kd.shape[1]
    cache = fam.ChunkedCache(B, Hq, Hkv, d, chunk, budget, sinks, W, kd.dtype, DEV)
    for p0 in range(0, S, chunk):
        cache.append(kd[:, :, p0:p0 + chunk], vd[:, :, p0:p0 + chunk])
        lse, mass = cache.score(qd[:, :, p0:p0 + chunk])
        if p0 + chunk < S:
            cache.compress()
    torch.cuda.synchronize()
    n = cache.n
    assert n == budget + chunk
    pos = cache.pos[:, :n].cpu().numpy().astype(np.int64)
    assert np.all(np.diff(pos, axis=1) > 0)
    assert np.all(pos[:, :sinks] == np.arange(sinks)) and np.all(pos[:, -chunk - W:] == np.arange(S - chunk - W, S))
    p0 = S - chunk
    grp, tail = 5, 64
    g = Hq // Hkv
    kh = cache.k[grp, :n].cpu().to(torch.float64).numpy()[None]
    qg = t["q"][0, grp * g:(grp + 1) * g, p0:].to(torch.float64).numpy()
    P = pos[grp:grp + 1]
    rows = np.sort(np.random.default_rng(0).choice(chunk, 48, replace=False))
    rows = np.concatenate([rows, np.arange(chunk - tail, chunk)])
    lse_got = to64(lse[0, grp * g:(grp + 1) * g])
    for qi in range(g):
        # normalisers of sampled rows (positions p0 + r)
        ref = np.array([ch.chunk_lse(qg[qi:qi + 1, r:r + 1], kh, P, p0 + r)[0, 0] for r in rows])
        check_lse(lse_got[qi, rows], ref)
    # keys counted only by the last `tail` queries: rows n - W - tail .. n - W - 1
    keys = np.arange(n - W - tail, n - W)
    lse_tail = np.stack([ch.chunk_lse(qg[qi:qi + 1, chunk - tail:], kh, P, S - tail)[0] for qi in range(g)])
    want = np.zeros(keys.size)
    for qi in range(g):
        m = ch.chunk_mass(qg[qi:qi + 1, chunk - tail:], kh[:, keys], P[:, keys], lse_tail[qi:qi + 1],
                          S - tail, W)
        want += m[0]
    check_mass(to64(mass[0, grp])[keys], want)
