"""Debug switches and the bounded wait of the in-place compaction.

* FAM_SYNC_CHECK=1: every device entry point synchronises and reports the
  outcome of the work it enqueued; the normal path still gives the same
  results bit for bit.
* The in-place compaction's waits are bounded. When a wait runs out of
  polls the chunk leaves its rows unwritten and counts itself in the
  workspace's error word, which kv_compact_inplace_status reports as
  FAM_ERR_TIMEOUT (and kv_compact_inplace itself under FAM_SYNC_CHECK). The
  test forces that path from the host with FAM_INPLACE_SPIN_LIMIT=0 (every
  wait gives up before its first poll), so every kernel still exits
  normally; then the same call without the limit moves every row.
"""
import os

import numpy as np
import pytest
import torch

from future_attention_scoring_amd import fam

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"\n[case] {msg}", flush=True)


class env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def shifted_case(seed):
    """Two heads whose kept rows lie far after their outputs, so that almost
    every chunk has earlier chunks to wait for."""
    H, S, d = 2, 20000, 128
    g = torch.Generator(device=DEV).manual_seed(seed)
    k = torch.randn(H, S, d, device=DEV, generator=g).to(torch.bfloat16)
    v = torch.randn(H, S, d, device=DEV, generator=g).to(torch.bfloat16)
    keeps = [np.concatenate([np.arange(4), np.arange(9004, S)]), np.arange(5000, S, 2)]
    idx = torch.from_numpy(np.concatenate(keeps).astype(np.int32)).to(DEV)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum([len(x) for x in keeps])]).astype(np.int64)).to(DEV)
    return k, v, keeps, idx, off


def test_inplace_timeout_is_reported_and_the_normal_path_completes():
    say("kv_compact_inplace with FAM_INPLACE_SPIN_LIMIT=0, then without")
    k, v, keeps, idx, off = shifted_case(1)
    k0, v0 = k.clone(), v.clone()
    ws = torch.empty(fam.kv_compact_inplace_workspace_size(idx.numel()), dtype=torch.uint8, device=DEV)
    with env(FAM_INPLACE_SPIN_LIMIT=0):
        fam.kv_compact_inplace(k, v, idx, off, workspace=ws)
    with pytest.raises(fam.FamError) as e:
        fam.kv_compact_inplace_status(ws)
    assert e.value.status == 5 and "gave up" in e.value.detail
    # the first chunk (256 rows at d = 128) waits for nobody and moved its
    # rows; every later chunk of head 0 waits for it, gave up and left its
    # rows as they were
    keep0 = torch.from_numpy(keeps[0][:256].astype(np.int64)).to(DEV)
    assert torch.equal(k[0, :256].view(torch.int16), k0[0, keep0].view(torch.int16))
    assert torch.equal(k[0, 256:1000].view(torch.int16), k0[0, 256:1000].view(torch.int16))

    k, v, keeps, idx, off = shifted_case(1)
    fam.kv_compact_inplace(k, v, idx, off, workspace=ws)
    fam.kv_compact_inplace_status(ws)                    # no error
    for h, keep in enumerate(keeps):
        src = torch.from_numpy(keep.astype(np.int64)).to(DEV)
        assert torch.equal(k[h, :len(keep)].view(torch.int16), k0[h, src].view(torch.int16)), h
        assert torch.equal(v[h, :len(keep)].view(torch.int16), v0[h, src].view(torch.int16)), h


def test_sync_check_reports_the_timeout_from_the_call_itself():
    say("FAM_SYNC_CHECK=1 with FAM_INPLACE_SPIN_LIMIT=0")
    k, v, keeps, idx, off = shifted_case(2)
    with env(FAM_SYNC_CHECK=1, FAM_INPLACE_SPIN_LIMIT=0):
        with pytest.raises(fam.FamError) as e:
            fam.kv_compact_inplace(k, v, idx, off)
    assert e.value.status == 5


def test_sync_check_leaves_results_unchanged():
    say("FAM_SYNC_CHECK=1: the path end to end, bit for bit against the normal run")
    B, Hq, Hkv, S, d, W = 1, 8, 2, 3000, 128, 64
    g = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn(B, Hq, S, d, device=DEV, generator=g).to(torch.bfloat16)
    kk = torch.randn(B, Hkv, S, d, device=DEV, generator=g).to(torch.bfloat16)
    vv = torch.randn(B, Hkv, S, d, device=DEV, generator=g).to(torch.bfloat16)

    def run():
        lse, mass = fam.fam_compute(q, kk, W)
        idx, off = fam.evict_select(mass[0], [700, 1500], 4, W)
        kn, vn = fam.kv_compact(kk[0], vv[0], idx, off)
        order = fam.fam_rank_order(mass[0])
        tau = fam.fam_topk_cutoff(order, 4, W, 300)
        ratio = fam.fam_eviction_cost_ratio(mass[0], mass[0])
        torch.cuda.synchronize()
        return [x.clone() for x in (lse, mass, idx, off, kn, vn, order, tau, ratio)]

    want = run()
    with env(FAM_SYNC_CHECK=1):
        got = run()
    for a, b in zip(want, got):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
