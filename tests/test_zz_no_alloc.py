"""evict_select_noalloc (the selection with the library's static device
scratch instead of a caller workspace) against evict_select, through the C
ABI: identical index lists and offsets, bit for bit, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's
contents), and a clear error for a size beyond the scratch array.
"""
import ctypes

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def noalloc_raw(scores, budgets, sinks, recent):
    """One call of the exported symbol with plain pointers."""
    H, S = scores.shape
    b = np.ascontiguousarray(budgets, dtype=np.int64)
    _, off = fam.evict_plan(b, S, sinks, recent)
    idx = torch.full((int(off[-1]),), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((H + 1,), -7, dtype=torch.int64, device=DEV)
    lib = fam.load()
    st = lib.evict_select_noalloc(ctypes.c_void_p(scores.data_ptr()), ctypes.c_int64(scores.stride(0)), H, S,
                                  b.ctypes.data_as(ctypes.c_void_p), sinks, recent,
                                  ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(offsets.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, idx, offsets


def test_noalloc_select_matches_evict_select_twice_then_smaller():
    rng = np.random.default_rng(31)
    wl = workloads.llama31_8b_128k()
    budgets = fam.fam_budgets_from_ratios(wl.ratios, wl.S).tolist()
    say(f"evict_select_noalloc: 8 heads x {wl.S}, then 56 heads x 4096")
    big = torch.from_numpy(rng.exponential(size=(8, wl.S)).astype(np.float32)).to(DEV)
    big[:, rng.random(wl.S) < 0.01] = 0.5                       # ties
    st, idx, off = noalloc_raw(big, budgets, wl.sinks, wl.recent)
    assert st == 0, fam.load().fam_last_error()
    ref_idx, ref_off = fam.evict_select(big, budgets, wl.sinks, wl.recent)
    torch.cuda.synchronize()
    assert torch.equal(off, ref_off) and torch.equal(idx, ref_idx)

    small = torch.from_numpy(rng.exponential(size=(56, 4096)).astype(np.float32)).to(DEV)
    bud = [int(x) for x in rng.integers(0, 4200, 56)]
    st, idx, off = noalloc_raw(small, bud, 4, 32)
    assert st == 0, fam.load().fam_last_error()
    ref_idx, ref_off = fam.evict_select(small, bud, 4, 32)
    torch.cuda.synchronize()
    assert torch.equal(off, ref_off) and torch.equal(idx, ref_idx)

    # the same small call once more through the binding: unchanged
    idx2 = torch.empty_like(idx)
    off2 = torch.empty_like(off)
    fam.evict_select_noalloc(small, bud, 4, 32, idx2, off2)
    torch.cuda.synchronize()
    assert torch.equal(idx2, ref_idx) and torch.equal(off2, ref_off)


def test_noalloc_select_rejects_sizes_beyond_its_scratch():
    say("evict_select_noalloc beyond its scratch array")
    H, S = 64, 131072 + 516
    need = fam.evict_select_workspace_size(H, S, 4, 512)
    assert need > (64 << 20)
    scores = torch.zeros((H, S), dtype=torch.float32, device=DEV)
    st, idx, off = noalloc_raw(scores, [1000] * H, 4, 512)
    assert st == 2 and "static array" in fam.load().fam_last_error().decode()
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and bool((off == -7).all())   # nothing written
