"""Guard regions around every output and workspace of every device entry point.

There is no GPU address sanitizer here, so out-of-bounds writes are caught
the plain way: each output and each workspace is a view into the middle of a
larger buffer whose bytes are all set to a sentinel; after the call the
bytes before and after the view must still hold the sentinel, and outputs
the ABI declares fully overwritten must hold no sentinel word any more.
Shapes are ragged (sequence lengths off every tile size, odd head counts,
unaligned row counts) and cover the split and range modes of the score
passes, the one-chunk and multi-chunk select, and the wavelet-matrix build.
Every call goes through the Python binding, i.e. the C ABI.
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096                  # bytes on each side (keeps 256-byte alignment of the view)
SENT = 0xA7                   # sentinel byte
SENT_WORD = {1: 0xA7, 2: 0xA7A7, 4: 0xA7A7A7A7, 8: 0xA7A7A7A7A7A7A7A7}


def say(msg):
    print(f"\n[case] {msg}", flush=True)


class Guarded:
    """A tensor view of `shape` and `dtype` inside sentinel-filled guard bytes."""

    def __init__(self, shape, dtype, full_overwrite=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        esize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * esize
        self.esize = esize
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), SENT, dtype=torch.uint8, device=DEV)
        inner = self.buf[GUARD:GUARD + self.nbytes]
        self.t = inner.view(dtype).view(self.shape) if self.nbytes else torch.empty(self.shape, dtype=dtype,
                                                                                      device=DEV)
        self.full = full_overwrite

    def check(self, name):
        torch.cuda.synchronize()
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        assert bool((head == SENT).all()), f"{name}: write before the output"
        assert bool((tail == SENT).all()), f"{name}: write after the output"
        if self.full and self.nbytes:
            words = self.buf[GUARD:GUARD + self.nbytes].view(
                {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[self.esize])
            sent = np.array(SENT_WORD[self.esize], dtype=np.uint64).astype(
                {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[self.esize]).view(
                {1: np.int8, 2: np.int16, 4: np.int32, 8: np.int64}[self.esize])
            left = int((words == int(sent)).sum())
            assert left == 0, f"{name}: {left} elements never written"


def ws(nbytes):
    return Guarded((max(int(nbytes), 0),), torch.uint8, full_overwrite=False)


SCORE_CASES = [
    # (B, Hq, Hkv, S, d, W)
    (1, 6, 2, 1000, 128, 37),
    (2, 3, 3, 259, 64, 0),
    (1, 4, 1, 65536 + 123, 128, 512),     # range mode of the mass pass, key-range split of pass 1
]


@pytest.mark.parametrize("B,Hq,Hkv,S,d,W", SCORE_CASES)
def test_score_entry_points_stay_inside_their_outputs(B, Hq, Hkv, S, d, W):
    say(f"guards: score passes B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} W={W}")
    g = torch.Generator(device=DEV).manual_seed(S)
    q = torch.randn(B, Hq, S, d, device=DEV, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, d, device=DEV, generator=g).to(torch.bfloat16)

    lse, mass = Guarded((B, Hq, S), torch.float32), Guarded((B, Hkv, S), torch.float32)
    w = ws(fam.fam_compute_workspace_size(B, Hq, Hkv, S, S))
    fam.fam_compute(q, k, W, lse=lse.t, mass=mass.t, workspace=w.t)
    for n, x in (("fam_compute lse", lse), ("fam_compute mass", mass), ("fam_compute workspace", w)):
        x.check(n)

    kn = Guarded((B, Hkv, fam.fam_key_norm_parts(S)), torch.float32)
    fam.fam_key_norms(k, knorm=kn.t)
    kn.check("fam_key_norms")
    lse2 = Guarded((B, Hq, S), torch.float32)
    fam.fam_lse(q, k, lse=lse2.t, knorm=kn.t)
    lse2.check("fam_lse")
    mass2 = Guarded((B, Hkv, S), torch.float32)
    w2 = ws(fam.fam_mass_workspace_size(B, Hq, Hkv, S))
    fam.fam_mass(q, k, lse2.t, W, mass=mass2.t, workspace=w2.t)
    mass2.check("fam_mass")
    w2.check("fam_mass workspace")
    # the mass pass feeding the select (the fused launch when it splits)
    H, sinks, recent = B * Hkv, 4, W + 3
    budgets = [S // 3 + 7 * h for h in range(H)]
    _, off = fam.evict_plan(budgets, S, sinks, recent)
    mass4, idx4, offs4 = Guarded((B, Hkv, S), torch.float32), Guarded((int(off[-1]),), torch.int32), \
        Guarded((H + 1,), torch.int64)
    w5, w6 = ws(fam.fam_mass_workspace_size(B, Hq, Hkv, S)), ws(fam.evict_select_workspace_size(H, S, sinks, recent))
    fam.fam_mass_select(q, k, lse2.t, W, budgets, sinks, recent, mass=mass4.t, idx=idx4.t, offsets=offs4.t,
                        mass_workspace=w5.t, select_workspace=w6.t)
    for n, x in (("fam_mass_select mass", mass4), ("fam_mass_select idx", idx4),
                 ("fam_mass_select offsets", offs4), ("fam_mass_select mass workspace", w5),
                 ("fam_mass_select select workspace", w6)):
        x.check(n)
    mq = Guarded((B, Hq, S), torch.float32)
    w3 = ws(fam.fam_mass_per_head_workspace_size(B, Hq, Hkv, S))
    fam.fam_mass_per_head(q, k, lse2.t, W, mass_q=mq.t, workspace=w3.t)
    mq.check("fam_mass_per_head")
    w3.check("fam_mass_per_head workspace")
    tg = Guarded((B, Hkv, S), torch.float32)
    fam.fam_kvpop_target(mq.t, Hkv, W, eps=1e-6, aggregate="max", target=tg.t)
    tg.check("fam_kvpop_target")

    Sq = min(S, 333)
    lse3, mass3 = Guarded((B, Hq, Sq), torch.float32), Guarded((B, Hkv, S), torch.float32)
    w4 = ws(fam.fam_compute_workspace_size(B, Hq, Hkv, Sq, S))
    fam.fam_compute_chunk(q[:, :, S - Sq:], k, W, lse=lse3.t, mass=mass3.t, workspace=w4.t)
    for n, x in (("chunk lse", lse3), ("chunk mass", mass3), ("chunk workspace", w4)):
        x.check(n)


@pytest.mark.parametrize("H,S,sinks,recent", [(5, 5000, 4, 64), (7, 3001, 4, 32), (3, 100001, 4, 512),
                                              (3, 150001, 4, 512)])
def test_eviction_entry_points_stay_inside_their_outputs(H, S, sinks, recent):
    say(f"guards: select/compact/ranking H={H} S={S}")
    rng = np.random.default_rng(S)
    scores = torch.from_numpy(rng.standard_normal((H, S)).astype(np.float32)).to(DEV)
    budgets = [int(b) for b in rng.integers(0, S + 10, H)]
    budgets[0] = 1                                   # below the forced set
    _, off = fam.evict_plan(budgets, S, sinks, recent)
    total = int(off[-1])
    idx, offs = Guarded((total,), torch.int32), Guarded((H + 1,), torch.int64)
    w = ws(fam.evict_select_workspace_size(H, S, sinks, recent))
    fam.evict_select(scores, budgets, sinks, recent, idx=idx.t, offsets=offs.t, workspace=w.t)
    idx.check("evict_select idx")
    offs.check("evict_select offsets")
    w.check("evict_select workspace")

    d = 128
    # non-negative rows: no 2-byte element equals the (negative) sentinel word
    kc = torch.randn(H, S, d, device=DEV).abs().to(torch.float16)
    vc = torch.randn(H, S, d, device=DEV).abs().to(torch.float16)
    kn, vn = Guarded((total, d), torch.float16), Guarded((total, d), torch.float16)
    fam.kv_compact(kc, vc, idx.t, offs.t, total_rows=total, k_new=kn.t, v_new=vn.t)
    kn.check("kv_compact k_new")
    vn.check("kv_compact v_new")

    order = Guarded((H, S), torch.int32)
    w = ws(fam.fam_rank_order_workspace_size(H, S))
    fam.fam_rank_order(scores, order=order.t, workspace=w.t)
    order.check("fam_rank_order")
    w.check("fam_rank_order workspace")
    imp = scores.abs()
    cost = Guarded((H,), torch.float64)
    w = ws(fam.fam_eviction_cost_workspace_size(H, S))
    fam.fam_eviction_cost(imp, order.t, cost=cost.t, workspace=w.t)
    cost.check("fam_eviction_cost")
    w.check("fam_eviction_cost workspace")
    ratio = Guarded((H,), torch.float64)
    w = ws(fam.fam_eviction_cost_ratio_workspace_size(H, S))
    fam.fam_eviction_cost_ratio(scores, imp, ratio=ratio.t, workspace=w.t)
    ratio.check("fam_eviction_cost_ratio")
    w.check("fam_eviction_cost_ratio workspace")
    common = Guarded((H,), torch.int64)
    fam.fam_retention_overlap(idx.t, offs.t, idx.t, offs.t, S, common=common.t)
    common.check("fam_retention_overlap")
    tau = Guarded((H, S), torch.int32)
    w = ws(fam.fam_topk_cutoff_workspace_size(H, S))
    fam.fam_topk_cutoff(order.t, sinks, recent, max(1, S // 9), tau=tau.t, workspace=w.t)
    tau.check("fam_topk_cutoff")
    w.check("fam_topk_cutoff workspace")


def test_cache_entry_points_write_only_their_rows():
    """kv_append writes rows row0 .. row0+n-1 (and their positions) only;
    kv_compact_inplace writes rows below each head's kept count only, and its
    workspace stays inside its size."""
    H, cap, d, n, row0 = 3, 3000, 128, 777, 1100
    say(f"guards: kv_append / kv_compact_inplace H={H} capacity={cap}")
    kc = Guarded((H, cap, d), torch.bfloat16, full_overwrite=False)
    vc = Guarded((H, cap, d), torch.bfloat16, full_overwrite=False)
    pos = Guarded((H, cap), torch.int32, full_overwrite=False)
    ks = torch.randn(H, n, d, device=DEV).to(torch.bfloat16)
    vs = torch.randn(H, n, d, device=DEV).to(torch.bfloat16)
    before_k = kc.t.clone()
    fam.kv_append(ks, vs, kc.t, vc.t, row0, pos=pos.t, pos0=5000)
    for name, x in (("kv_append k", kc), ("kv_append v", vc), ("kv_append pos", pos)):
        x.check(name)
    rows = torch.ones(cap, dtype=torch.bool, device=DEV)
    rows[row0:row0 + n] = False
    assert torch.equal(kc.t[:, rows].view(torch.int16), before_k[:, rows].view(torch.int16))
    assert torch.equal(kc.t[:, row0:row0 + n], ks)
    assert torch.equal(pos.t[:, row0:row0 + n].cpu(), torch.arange(5000, 5000 + n, dtype=torch.int32).expand(H, n))

    rng = np.random.default_rng(3)
    keeps = [np.sort(rng.choice(cap, size=m, replace=False)) for m in (1500, 0, 2999)]
    idx = torch.from_numpy(np.concatenate(keeps).astype(np.int32)).to(DEV)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum([len(x) for x in keeps])]).astype(np.int64)).to(DEV)
    total = int(offsets[-1])
    before_k = kc.t.clone()
    w = ws(fam.kv_compact_inplace_workspace_size(total))
    fam.kv_compact_inplace(kc.t, vc.t, idx, offsets, pos=pos.t, workspace=w.t)
    for name, x in (("inplace k", kc), ("inplace v", vc), ("inplace pos", pos), ("inplace workspace", w)):
        x.check(name)
    for h, keep in enumerate(keeps):
        m = len(keep)
        assert torch.equal(kc.t[h, m:].view(torch.int16), before_k[h, m:].view(torch.int16)), h
        src = torch.from_numpy(keep.astype(np.int64)).to(DEV)
        assert torch.equal(kc.t[h, :m].view(torch.int16), before_k[h, src].view(torch.int16)), h
