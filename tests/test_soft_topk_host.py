"""The library's host-side Soft-TopK (fam_soft_topk, C++) against the pinned
fp64 oracle (oracle/soft_topk.py), plus the operator's stated properties
checked on the library itself: sums to k, order preserved, shift invariant,
softmax-like at k = 1 when no weight reaches one half, hard top-k as tau -> 0.
CPU only: the function runs on the host.
"""
import numpy as np
import pytest

from future_attention_scoring_amd import fam
from oracle import soft_topk as st


@pytest.mark.parametrize("seed,n,k,tau", [(0, 2, 1.0, 1.0), (1, 10, 3.0, 1.0), (2, 56, 8.4, 0.5),
                                          (3, 1000, 150.0, 2.0), (4, 64, 63.5, 1.0), (5, 7, 0.25, 0.1)])
def test_matches_oracle(seed, n, k, tau):
    x = np.random.default_rng(seed).standard_normal(n) * 3
    got = fam.fam_soft_topk(x, k, tau)
    np.testing.assert_allclose(got, st.soft_topk(x, k, tau), rtol=1e-11, atol=1e-14)


def test_properties():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(200)
    m = fam.fam_soft_topk(x, 20.0)
    assert abs(m.sum() - 20.0) < 1e-9
    assert np.all((m > 0) & (m < 1))
    order = np.argsort(-x)
    assert np.all(np.diff(m[order]) <= 1e-15)
    np.testing.assert_allclose(fam.fam_soft_topk(x + 7.5, 20.0), m, rtol=1e-10, atol=1e-13)
    # hard top-k as tau -> 0 (entries 0.05 apart: the mask is within e^-25 of 0 or 1)
    y = rng.permutation(np.arange(200) * 0.05)
    hard = fam.fam_soft_topk(y, 20.0, tau=1e-3)
    top = np.zeros_like(y)
    top[np.argsort(-y)[:20]] = 1.0
    np.testing.assert_allclose(hard, top, atol=1e-9)


def test_k1_is_softmax_when_no_weight_reaches_half():
    x = np.random.default_rng(2).standard_normal(50) * 0.3
    m = fam.fam_soft_topk(x, 1.0)
    e = np.exp(x - x.max())
    np.testing.assert_allclose(m, e / e.sum(), rtol=1e-12)


def test_lkv_head_budgets_pipeline():
    scores = np.random.default_rng(4).standard_normal((28, 2))     # layers x KV heads
    r = fam.fam_soft_topk(scores, 0.15 * scores.size)
    np.testing.assert_allclose(r, st.head_ratios(scores, 0.15), rtol=1e-11)
    b = fam.fam_budgets_from_ratios(r.ravel(), 131072)
    assert b.tolist() == st.head_budgets(r.ravel(), 131072).tolist()


def test_rejects_bad_arguments():
    for args in (([1.0, 2.0], 0.0), ([1.0, 2.0], 2.0), ([np.nan, 1.0], 1.0)):
        with pytest.raises(fam.FamError):
            fam.fam_soft_topk(*args)
    with pytest.raises(fam.FamError):
        fam.fam_soft_topk([1.0, 2.0], 1.0, tau=0.0)
