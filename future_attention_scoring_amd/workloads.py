"""Seeded synthetic inputs for the future-attention-mass and eviction path.

This module only draws random tensors. It holds none of the method's
arithmetic (no softmax, no mass, no budget floor, no selection), so the
oracle and the HIP path can both consume its output without sharing any
computation.

Every tensor is drawn per head from its own numpy ``default_rng`` stream
keyed by ``(seed, tag, head)``, so a single head can be regenerated without
drawing the rest (the oracle's samples of the 128k workload rely on that).
Values are drawn in fp32 and rounded to the storage dtype with torch's
round-to-nearest-even conversion; the oracle reads the rounded values.

The workloads stand in for real activations of the models the pages
evaluate on (KVpop: Qwen3-4B/8B reasoning traces; LKV: Llama-3.1-8B on
LongBench; the pruning blog: Qwen2.5-1.5B caches). No dataset item is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_TAGS = {"q": 1, "k": 2, "v": 3, "u": 4, "hot": 5, "mix": 6, "score": 7, "ratio": 8}


def _rng(seed: int, tag: str, head: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TAGS[tag], int(head)])


def normal_heads(seed: int, tag: str, heads: Sequence[int], S: int, d: int) -> np.ndarray:
    """N(0,1) fp32 rows ``[len(heads), S, d]``, one stream per head."""
    out = np.empty((len(heads), S, d), dtype=np.float32)
    for n, h in enumerate(heads):
        out[n] = _rng(seed, tag, h).standard_normal((S, d), dtype=np.float32)
    return out


def _unit(seed: int, tag: str, head: int, d: int) -> np.ndarray:
    u = _rng(seed, tag, head).standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp32 numpy -> torch tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


@dataclasses.dataclass
class ScoreWorkload:
    """One fam_compute -> evict_select -> kv_compact workload (batch 1)."""

    name: str
    seed: int
    Hq: int
    Hkv: int
    S: int
    d: int
    W: int
    sinks: int
    recent: int
    dtype: torch.dtype = torch.bfloat16
    # uniform total budget per KV head, or None when ``ratios`` give budgets
    budget: Optional[int] = None
    # per-KV-head retention ratios r_h (budgets are floor(r_h * S))
    ratios: Optional[np.ndarray] = None
    # "plain": Q,K ~ N(0,1); "hot": rank-1 per-head hot-key bias;
    # "mixture": 10% of keys shifted by +2 sigma along one shared direction
    kind: str = "plain"

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def q_heads(self, heads: Sequence[int]) -> np.ndarray:
        """fp32 queries for the listed query heads, ``[n, S, d]``."""
        q = normal_heads(self.seed, "q", heads, self.S, self.d)
        if self.kind == "hot":
            alpha = math.sqrt(3.0 * math.sqrt(self.d))
            for n, h in enumerate(heads):
                q[n] += alpha * _unit(self.seed, "u", h // self.group, self.d)[None, :]
        return q

    def k_heads(self, heads: Sequence[int]) -> np.ndarray:
        """fp32 keys for the listed KV heads, ``[n, S, d]``."""
        k = normal_heads(self.seed, "k", heads, self.S, self.d)
        if self.kind == "hot":
            alpha = math.sqrt(3.0 * math.sqrt(self.d))
            for n, h in enumerate(heads):
                hot = _rng(self.seed, "hot", h).random(self.S) < 0.05
                k[n, hot] += alpha * _unit(self.seed, "u", h, self.d)[None, :]
        elif self.kind == "mixture":
            u = _unit(self.seed, "u", 0, self.d)
            for n, h in enumerate(heads):
                shifted = _rng(self.seed, "mix", h).random(self.S) < 0.10
                k[n, shifted] += 2.0 * u[None, :]
        return k

    def v_heads(self, heads: Sequence[int]) -> np.ndarray:
        return normal_heads(self.seed, "v", heads, self.S, self.d)

    def tensors(self, q_heads: Optional[Sequence[int]] = None,
                kv_heads: Optional[Sequence[int]] = None,
                with_v: bool = True) -> Dict[str, torch.Tensor]:
        """CPU tensors ``q [1,nq,S,d]``, ``k``/``v [1,nkv,S,d]`` in ``dtype``."""
        qh = list(range(self.Hq)) if q_heads is None else list(q_heads)
        kh = list(range(self.Hkv)) if kv_heads is None else list(kv_heads)
        out = {"q": to_dtype(self.q_heads(qh), self.dtype).unsqueeze(0),
               "k": to_dtype(self.k_heads(kh), self.dtype).unsqueeze(0)}
        if with_v:
            out["v"] = to_dtype(self.v_heads(kh), self.dtype).unsqueeze(0)
        return out

    def budget_inputs(self) -> Dict[str, object]:
        """What budgets derive from: a uniform total, or ratios and t = S."""
        if self.ratios is not None:
            return {"ratios": self.ratios.copy(), "t": self.S}
        return {"uniform": int(self.budget)}


def dirichlet_ratios(seed: int, n: int, mean: float) -> np.ndarray:
    """Per-head ratios ``n * mean * Dirichlet(1_n)`` (their mean is ``mean``)."""
    return n * mean * _rng(seed, "ratio", 0).dirichlet(np.ones(n))


def tiny(seed: int = 1) -> ScoreWorkload:
    """S=512, d=64, 2 query heads = 2 KV heads, W=32, 4 sinks, 128 kept."""
    return ScoreWorkload("tiny-s512-d64", seed, Hq=2, Hkv=2, S=512, d=64, W=32,
                         sinks=4, recent=32, budget=128)


def qwen3_4b_layer(seed: int = 2, S: int = 8192) -> ScoreWorkload:
    """Qwen3-4B-like layer: 32 Q / 8 KV heads, d=128, ~5% hot keys, keep 2048."""
    return ScoreWorkload(f"qwen3-4b-layer-s{S}", seed, Hq=32, Hkv=8, S=S, d=128,
                         W=128, sinks=4, recent=128, budget=2048, kind="hot")


def long_trace(seed: int = 3, S: int = 32768) -> ScoreWorkload:
    """Long reasoning trace: mixture keys, W=256, keep 3932 per KV head."""
    return ScoreWorkload(f"long-trace-s{S}", seed, Hq=32, Hkv=8, S=S, d=128,
                         W=256, sinks=4, recent=256, budget=3932, kind="mixture")


def llama31_8b_128k(seed: int = 4, S: int = 131072) -> ScoreWorkload:
    """Llama-3.1-8B-like layer at 128k: W=512, Dirichlet per-head ratios."""
    return ScoreWorkload(f"llama3.1-8b-layer-s{S}", seed, Hq=32, Hkv=8, S=S,
                         d=128, W=512, sinks=4, recent=512,
                         ratios=dirichlet_ratios(seed, 8, 0.15))


@dataclasses.dataclass
class DecodeCell:
    """One cell of the decode-time eviction sweep (given scores, no fam)."""

    seed: int
    S: int
    budget: int
    layers: int = 28
    kv_heads: int = 2
    d: int = 128
    sinks: int = 4
    recent: int = 32
    dtype: torch.dtype = torch.float16

    @property
    def H(self) -> int:
        return self.layers * self.kv_heads

    def scores(self) -> np.ndarray:
        """fp32 per-token scores ``[H, S]`` ~ Exp(1)."""
        out = np.empty((self.H, self.S), dtype=np.float32)
        for h in range(self.H):
            out[h] = _rng(self.seed, "score", h).exponential(size=self.S).astype(np.float32)
        return out

    def kv(self) -> Dict[str, torch.Tensor]:
        heads = range(self.H)
        return {"k": to_dtype(normal_heads(self.seed, "k", heads, self.S, self.d), self.dtype),
                "v": to_dtype(normal_heads(self.seed, "v", heads, self.S, self.d), self.dtype)}


DECODE_CONTEXTS: List[int] = [512, 4096, 32768, 120000]
DECODE_BUDGETS: List[int] = [4096, 2048, 1024, 512]


def decode_sweep(seed: int = 5) -> List[DecodeCell]:
    """Qwen2.5-1.5B-like cache (28 layers x 2 KV heads, d=128, fp16)."""
    return [DecodeCell(seed, S, b) for S in DECODE_CONTEXTS for b in DECODE_BUDGETS]
