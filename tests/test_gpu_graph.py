"""The hot path captured in a HIP graph and replayed.

One step of the path (key norms, first pass, mass pass, evict_select,
kv_compact), the same step with fam_mass_select, and one compression of the
chunked loop (evict_select, kv_compact_inplace with its fill kernel) are
captured with
torch.cuda.graph and replayed several times, with eager work of the same
kernels and synchronisations between the replays. Every replay must equal
the eager result bit for bit, also after the inputs were overwritten in
place between replays (the graph reads its inputs live). The library records
no memset: buffers it needs cleared are cleared by its own fill kernels, and
the per-head select parameters travel in the kernel arguments.
"""
import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def seeded(seed, shape, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype).to(DEV)


def test_score_select_compact_step_in_a_graph():
    B, Hq, Hkv, S, d, W, sinks, recent = 1, 8, 2, 3000, 128, 64, 4, 64
    budgets = [800, 1500]
    say(f"graph: fam_compute + evict_select + kv_compact S={S}")
    q, k, v = seeded(1, (B, Hq, S, d)), seeded(2, (B, Hkv, S, d)), seeded(3, (B, Hkv, S, d))
    lse = torch.empty(B, Hq, S, device=DEV)
    mass = torch.empty(B, Hkv, S, device=DEV)
    ws = torch.empty(max(16, fam.fam_compute_workspace_size(B, Hq, Hkv, S, S)), dtype=torch.uint8, device=DEV)
    _, host_off = fam.evict_plan(budgets, S, sinks, recent)
    total = int(host_off[-1])
    idx = torch.empty(total, dtype=torch.int32, device=DEV)
    offsets = torch.empty(Hkv + 1, dtype=torch.int64, device=DEV)
    sel_ws = torch.empty(max(16, fam.evict_select_workspace_size(Hkv, S, sinks, recent)), dtype=torch.uint8,
                         device=DEV)
    k_new = torch.empty(total, d, dtype=k.dtype, device=DEV)
    v_new = torch.empty_like(k_new)

    def step():
        fam.fam_compute(q, k, W, lse=lse, mass=mass, workspace=ws)
        fam.evict_select(mass[0], budgets, sinks, recent, idx=idx, offsets=offsets, workspace=sel_ws)
        fam.kv_compact(k[0], v[0], idx, offsets, total_rows=total, k_new=k_new, v_new=v_new)

    def snapshot():
        return [t.clone() for t in (lse, mass, idx, offsets, k_new, v_new)]

    step()
    torch.cuda.synchronize()
    want = snapshot()

    # warm the capture stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (lse, mass, k_new, v_new):
            t.fill_(0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int8) if b.dtype == torch.bfloat16 else b), f"replay {rep}"
        # eager work of the same kernels on other data between replays
        fam.fam_compute(seeded(10 + rep, (B, Hq, S, d)), seeded(20 + rep, (B, Hkv, S, d)), W)
        torch.cuda.synchronize()

    # new inputs in place: the replay must follow them
    q.copy_(seeded(7, (B, Hq, S, d)))
    k.copy_(seeded(8, (B, Hkv, S, d)))
    step()
    torch.cuda.synchronize()
    want2 = snapshot()
    assert not torch.equal(want2[1], want[1])
    for t in (lse, mass, k_new, v_new):
        t.fill_(0)
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(snapshot(), want2):
        assert torch.equal(a.view(torch.int8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int8) if b.dtype == torch.bfloat16 else b), "replay after new inputs"


def test_inplace_compression_and_cutoff_in_a_graph():
    H, S, d, keep, sinks, recent = 4, 5000, 128, 3000, 4, 128
    say(f"graph: evict_select + kv_compact_inplace, rank order + cut-off H={H} S={S}")
    scores = torch.rand(H, S, generator=torch.Generator().manual_seed(5)).to(DEV)
    k0, v0 = seeded(11, (H, S, d)), seeded(12, (H, S, d))
    k, v = k0.clone(), v0.clone()
    budgets = [keep] * H
    _, host_off = fam.evict_plan(budgets, S, sinks, recent)
    total = int(host_off[-1])
    idx = torch.empty(total, dtype=torch.int32, device=DEV)
    offsets = torch.empty(H + 1, dtype=torch.int64, device=DEV)
    sel_ws = torch.empty(max(16, fam.evict_select_workspace_size(H, S, sinks, recent)), dtype=torch.uint8,
                         device=DEV)
    ip_ws = torch.empty(fam.kv_compact_inplace_workspace_size(total), dtype=torch.uint8, device=DEV)
    order = torch.empty(H, S, dtype=torch.int32, device=DEV)
    rank_ws = torch.empty(max(8, fam.fam_rank_order_workspace_size(H, S)), dtype=torch.uint8, device=DEV)
    tau = torch.empty(H, S, dtype=torch.int32, device=DEV)
    cut_ws = torch.empty(max(4, fam.fam_topk_cutoff_workspace_size(H, S)), dtype=torch.uint8, device=DEV)

    def step():
        fam.evict_select(scores, budgets, sinks, recent, idx=idx, offsets=offsets, workspace=sel_ws)
        fam.kv_compact_inplace(k, v, idx, offsets, total_rows=total, workspace=ip_ws)
        fam.fam_rank_order(scores, order=order, workspace=rank_ws)
        fam.fam_topk_cutoff(order, sinks, 16, 700, tau=tau, workspace=cut_ws)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (idx, offsets, k, v, order, tau)]
    off = offsets.cpu().tolist()
    idx_h = idx.cpu().numpy()
    for h in range(H):   # the eager in-place result is the gather of the kept rows
        rows = torch.from_numpy(idx_h[off[h]:off[h + 1]].astype(np.int64)).to(DEV)
        assert torch.equal(k[h, :off[h + 1] - off[h]].view(torch.int16), k0[h, rows].view(torch.int16))

    k.copy_(k0)
    v.copy_(v0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    k.copy_(k0)
    v.copy_(v0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        k.copy_(k0)
        v.copy_(v0)
        for t in (idx, order, tau):
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((idx, offsets, k, v, order, tau), want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"replay {rep}"
        # eager in-place compaction on other buffers between replays
        k2, v2 = k0.clone(), v0.clone()
        fam.kv_compact_inplace(k2, v2, idx, offsets, total_rows=total)
        torch.cuda.synchronize()


def test_combined_mass_select_step_in_a_graph():
    """The step with fam_mass_select (the mass pass's reduction building the
    select histograms) captured and replayed: every replay equals the eager
    result and the two-call form bit for bit."""
    B, Hq, Hkv, S, d, W, sinks, recent = 1, 8, 2, 9000, 128, 64, 4, 64
    budgets = [2500, 4100]
    say(f"graph: fam_lse + fam_mass_select + kv_compact S={S}")
    q, k, v = seeded(31, (B, Hq, S, d)), seeded(32, (B, Hkv, S, d)), seeded(33, (B, Hkv, S, d))
    knorm = torch.empty(B, Hkv, fam.fam_key_norm_parts(S), device=DEV)
    lse = torch.empty(B, Hq, S, device=DEV)
    mass = torch.empty(B, Hkv, S, device=DEV)
    mws = torch.empty(fam.fam_mass_workspace_size(B, Hq, Hkv, S), dtype=torch.uint8, device=DEV)
    assert mws.numel() > 0                    # the mass pass splits: the combined launch runs
    _, host_off = fam.evict_plan(budgets, S, sinks, recent)
    total = int(host_off[-1])
    idx = torch.empty(total, dtype=torch.int32, device=DEV)
    offsets = torch.empty(Hkv + 1, dtype=torch.int64, device=DEV)
    sws = torch.empty(max(16, fam.evict_select_workspace_size(Hkv, S, sinks, recent)), dtype=torch.uint8,
                      device=DEV)
    k_new = torch.empty(total, d, dtype=k.dtype, device=DEV)
    v_new = torch.empty_like(k_new)

    def step():
        fam.fam_key_norms(k, knorm=knorm)
        fam.fam_lse(q, k, lse=lse, knorm=knorm)
        fam.fam_mass_select(q, k, lse, W, budgets, sinks, recent, mass=mass, idx=idx, offsets=offsets,
                            mass_workspace=mws, select_workspace=sws)
        fam.kv_compact(k[0], v[0], idx, offsets, total_rows=total, k_new=k_new, v_new=v_new)

    def snapshot():
        return [t.clone() for t in (lse, mass, idx, offsets, k_new.view(torch.int16), v_new.view(torch.int16))]

    step()
    torch.cuda.synchronize()
    want = snapshot()
    ref_mass = fam.fam_mass(q, k, lse, W)
    ref_idx, ref_off = fam.evict_select(ref_mass[0], budgets, sinks, recent)
    torch.cuda.synchronize()
    assert torch.equal(ref_mass.view(torch.int32), want[1].view(torch.int32))
    assert torch.equal(ref_idx, want[2]) and torch.equal(ref_off, want[3])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (lse, mass, k_new, v_new):
            t.fill_(0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), want):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work of the same kernels on other data between replays
        q2, k2 = seeded(40 + rep, (B, Hq, S, d)), seeded(50 + rep, (B, Hkv, S, d))
        fam.fam_mass_select(q2, k2, fam.fam_lse(q2, k2), W, budgets, sinks, recent)
        torch.cuda.synchronize()
