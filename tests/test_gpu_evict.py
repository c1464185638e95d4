"""GPU parity of evict_select and kv_compact against the oracle (bit-exact).

Selection is compared on identical fp32 scores: the GPU's own mass (copied to
the host) or the decode sweep's given scores feed both the oracle's sort-based
selection and the GPU's radix selection, and the index lists must be equal.
Compaction must reproduce the oracle's fancy-index gather bit for bit.
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


def gpu_select(scores_np, budgets, sinks, recent):
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(DEV)
    idx, off = fam.evict_select(s, budgets, sinks, recent)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), off.cpu().numpy()


def assert_select_equal(scores_np, budgets, sinks, recent):
    idx, off = gpu_select(scores_np, budgets, sinks, recent)
    idx_ref, off_ref = so.select(scores_np, budgets, sinks, recent)
    assert off.tolist() == off_ref.tolist()
    assert np.array_equal(idx, idx_ref), "index lists differ"
    return idx, off


def nasty(rng, H, S):
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5, 1e-38, -1e-38, 3.0],
                    dtype=np.float32)
    s = rng.choice(pool, size=(H, S)).astype(np.float32)
    mix = rng.random((H, S)) < 0.5
    s[mix] = rng.standard_normal(mix.sum()).astype(np.float32)
    return s


@pytest.mark.parametrize("seed,H,S,sinks,recent", [
    (0, 3, 1, 4, 4), (1, 5, 37, 0, 0), (2, 4, 300, 4, 32), (3, 2, 5000, 4, 16),
    (4, 7, 4099, 1, 100), (5, 2, 70000, 4, 512), (6, 2, 131072 + 4 + 512, 4, 512),
    (7, 3, 600, 400, 400),
])
def test_select_random_and_special_values(seed, H, S, sinks, recent):
    say(f"select seed={seed} H={H} S={S}")
    rng = np.random.default_rng(seed)
    scores = nasty(rng, H, S)
    budgets = [int(x) for x in rng.integers(0, S + 8, H)]
    budgets[0] = sinks + recent + 1
    assert_select_equal(scores, budgets, sinks, recent)


def test_select_ties_and_degenerate_budgets():
    say("ties / degenerate budgets")
    S = 9000
    scores = np.zeros((6, S), dtype=np.float32)
    scores[1] = np.arange(S, dtype=np.float32)          # sinks + newest
    scores[2, ::3] = 1.0                                 # many ties at the threshold
    scores[3] = np.float32(-0.0)
    scores[3, ::2] = 0.0
    scores[4] = np.nan
    scores[5] = np.repeat(np.arange(S // 100, dtype=np.float32), 100)
    budgets = [100, 500, 2999, 4000, 777, S + 100]
    idx, off = assert_select_equal(scores, budgets, 4, 32)
    head1 = idx[off[1]:off[2]]
    assert head1.tolist() == list(range(4)) + list(range(S - 496, S))
    assert_select_equal(scores, [0] * 6, 4, 32)                      # forced set only
    assert_select_equal(scores, [S] * 6, 4, 32)                      # everything


@pytest.mark.parametrize("budgets", [[0, 0, 0], [5000, 9000, 4096], [0, 4096, 1], [4096, 0, 70]])
def test_select_every_head_trivial(budgets):
    """Heads that keep only the forced rows or every row need no threshold;
    when all heads are such, only the last launch runs (the last two cases
    mix trivial heads with ones that need a threshold, so all three run)."""
    say(f"select with trivial heads {budgets}")
    S = 4096
    rng = np.random.default_rng(17)
    scores = rng.standard_normal((3, S)).astype(np.float32)
    assert_select_equal(scores, budgets, 4, 32)


def test_select_more_heads_than_a_batch():
    """150 heads run as batches of 64, 64 and 22 (the last batch's heads are
    offset into the same idx and offsets); some batches mix trivial heads
    (budget 0 or >= S) with ones that need a threshold, one batch has only
    trivial heads. Compaction of the result is checked too."""
    H, S, d = 150, 2000, 64
    say(f"select + compact H={H} S={S}")
    rng = np.random.default_rng(23)
    scores = nasty(rng, H, S)
    budgets = [int(x) for x in rng.integers(0, S + 8, H)]
    for h in range(64, 128):          # the second batch: trivial heads only
        budgets[h] = 0 if h % 2 else S + 5
    idx, off = assert_select_equal(scores, budgets, 4, 32)
    g = torch.Generator().manual_seed(23)
    k = torch.randn(H, S, d, generator=g).to(torch.float16)
    v = torch.randn(H, S, d, generator=g).to(torch.float16)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    off_d = torch.from_numpy(np.ascontiguousarray(off, dtype=np.int64)).to(DEV)
    k_new, v_new = fam.kv_compact(k.to(DEV), v.to(DEV), idx_d, off_d)
    torch.cuda.synchronize()
    o = np.asarray(off, dtype=np.int64)
    ih = np.asarray(idx, dtype=np.int64)
    kn, vn = k_new.cpu(), v_new.cpu()
    for h in range(H):
        rows = torch.from_numpy(ih[o[h]:o[h + 1]])
        assert torch.equal(kn[o[h]:o[h + 1]].view(torch.int16), k[h, rows].view(torch.int16))
        assert torch.equal(vn[o[h]:o[h + 1]].view(torch.int16), v[h, rows].view(torch.int16))


@pytest.mark.parametrize("seed,H,S,sinks,recent,kind", [
    (20, 8, 300000, 4, 512, "mass"), (21, 3, 131072 + 4 + 512 + 1, 4, 512, "nasty"),
    (22, 56, 150000, 4, 32, "exp"), (23, 2, (1 << 20) + 516, 4, 512, "ties"),
    (24, 4, 200003, 0, 0, "split"),
])
def test_select_beyond_131072_candidates(seed, H, S, sinks, recent, kind):
    """The round-based path (more than 131072 candidates a head): mass-like
    heavy-tailed scores with the 128k layer's Dirichlet budget mix at 300000
    positions x 8 heads, special values, Exp(1) scores over 56 heads (more
    heads than one launch holds), all-equal scores at the largest size (every
    key in one bin, lowest positions win), and scores with few distinct
    values so that the last level splits equal keys across chunks."""
    say(f"select long path seed={seed} H={H} S={S} {kind}")
    rng = np.random.default_rng(seed)
    if kind == "mass":
        scores = (rng.exponential(size=(H, S)) ** 3).astype(np.float32)
        ratios = 8 * 0.15 * rng.dirichlet(np.ones(H))
        budgets = [int(np.floor(r * S)) for r in ratios]
    elif kind == "nasty":
        scores = nasty(rng, H, S)
        budgets = [int(x) for x in rng.integers(0, S + 8, H)]
    elif kind == "exp":
        scores = rng.exponential(size=(H, S)).astype(np.float32)
        budgets = [4096, 2048, 1024, 512] * (H // 4)
    elif kind == "ties":
        scores = np.full((H, S), 0.5, dtype=np.float32)
        budgets = [S // 3, 777]
    else:
        scores = rng.integers(0, 3, size=(H, S)).astype(np.float32)
        budgets = [S // 2 + 1, S // 3, 100000, 5]
    assert_select_equal(scores, budgets, sinks, recent)


def test_select_unaligned_row_stride():
    say("unaligned score rows")
    rng = np.random.default_rng(9)
    H, S = 3, 1001
    buf = torch.from_numpy(rng.standard_normal((H, S + 3)).astype(np.float32)).to(DEV)
    view = buf[:, 1:S + 1]                                  # rows start at +4 bytes
    idx, off = fam.evict_select(view, [200, 300, 400], 4, 8)
    ref_idx, ref_off = so.select(view.cpu().numpy(), [200, 300, 400], 4, 8)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)


@pytest.mark.parametrize("wl_name", ["tiny", "qwen3_4b", "long_trace", "llama_128k"])
def test_select_on_gpu_mass_and_compact(wl_name):
    wl = {"tiny": workloads.tiny, "qwen3_4b": workloads.qwen3_4b_layer, "long_trace": workloads.long_trace,
          "llama_128k": workloads.llama31_8b_128k}[wl_name]()
    say(f"fam -> select -> compact {wl.name}")
    t = wl.tensors()
    q, k, v = t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV)
    _, mass = fam.fam_compute(q, k, wl.W)
    scores = mass[0].contiguous()
    bi = wl.budget_inputs()
    budgets = (so.budgets_from_ratios(bi["ratios"], bi["t"]).tolist() if "ratios" in bi
               else [bi["uniform"]] * wl.Hkv)
    idx, off = fam.evict_select(scores, budgets, wl.sinks, wl.recent)
    k_new, v_new = fam.kv_compact(k[0], v[0], idx, off)
    torch.cuda.synchronize()
    s_host = scores.cpu().numpy()
    idx_ref, off_ref = so.select(s_host, budgets, wl.sinks, wl.recent)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert off.cpu().numpy().tolist() == off_ref.tolist()
    k_ref = so.compact(t["k"][0].view(torch.int16).numpy(), idx_ref, off_ref)
    v_ref = so.compact(t["v"][0].view(torch.int16).numpy(), idx_ref, off_ref)
    assert np.array_equal(k_new.cpu().view(torch.int16).numpy(), k_ref)
    assert np.array_equal(v_new.cpu().view(torch.int16).numpy(), v_ref)


@pytest.mark.parametrize("S", workloads.DECODE_CONTEXTS)
def test_decode_sweep_select_compact(S):
    cells = [c for c in workloads.decode_sweep() if c.S == S]
    say(f"decode sweep S={S}")
    kv = cells[0].kv()
    k, v = kv["k"].to(DEV), kv["v"].to(DEV)
    scores = cells[0].scores()
    k16, v16 = kv["k"].view(torch.int16).numpy(), kv["v"].view(torch.int16).numpy()
    for cell in cells:
        budgets = [cell.budget] * cell.H
        idx, off = assert_select_equal(scores, budgets, cell.sinks, cell.recent)
        k_new, v_new = fam.kv_compact(k, v, torch.from_numpy(idx).to(DEV), torch.from_numpy(off).to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(k_new.cpu().view(torch.int16).numpy(), so.compact(k16, idx, off))
        assert np.array_equal(v_new.cpu().view(torch.int16).numpy(), so.compact(v16, idx, off))


def test_compact_identity_and_out_of_range_rows():
    say("compact identity / invalid index")
    H, S, d = 3, 257, 64
    k = torch.randn(H, S, d, dtype=torch.float16, device=DEV)
    v = torch.randn(H, S, d, dtype=torch.float16, device=DEV)
    idx = torch.arange(S, dtype=torch.int32, device=DEV).repeat(H)
    off = torch.tensor([0, S, 2 * S, 3 * S], dtype=torch.int64, device=DEV)
    k_new, v_new = fam.kv_compact(k, v, idx, off)
    assert torch.equal(k_new, k.reshape(-1, d)) and torch.equal(v_new, v.reshape(-1, d))
    bad = torch.tensor([0, -1, S, 5], dtype=torch.int32, device=DEV)
    off2 = torch.tensor([0, 2, 2, 4], dtype=torch.int64, device=DEV)
    k_new, _ = fam.kv_compact(k, v, bad, off2)
    assert torch.equal(k_new[0], k[0, 0]) and torch.equal(k_new[3], k[2, 5])
    assert torch.count_nonzero(k_new[1]) == 0 and torch.count_nonzero(k_new[2]) == 0


def test_select_deterministic():
    say("select determinism")
    rng = np.random.default_rng(11)
    scores = rng.exponential(size=(8, 50000)).astype(np.float32)
    a = gpu_select(scores, [5000] * 8, 4, 32)
    b = gpu_select(scores, [5000] * 8, 4, 32)
    assert np.array_equal(a[0], b[0])
