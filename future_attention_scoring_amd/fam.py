"""Thin ctypes binding over libfam.so (argument marshalling only).

Every function has the name of the C entry point it calls. Tensors are
torch tensors; torch supplies device memory and the current HIP stream, and
all computation happens in the library's HIP kernels. If libfam.so has not
been built the first call raises ``FamError``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfam.so")
_lib = None

FAM_BF16, FAM_FP16 = 0, 1
_STATUS = {0: "FAM_OK", 1: "FAM_ERR_INVALID_ARG", 2: "FAM_ERR_UNSUPPORTED",
           3: "FAM_ERR_WORKSPACE", 4: "FAM_ERR_HIP", 5: "FAM_ERR_TIMEOUT"}

# (name, restype, argtypes) of every exported symbol of include/fam.h
_i, _i64, _f, _p = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_SIGNATURES = {
    "fam_status_string": (ctypes.c_char_p, [_i]),
    "fam_last_error": (ctypes.c_char_p, []),
    "fam_key_norm_parts": (_i, [_i]),
    "fam_key_norms": (_i, [_p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _p, _p]),
    "fam_lse": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _i64, _f, _p, _p,
                     _p]),
    "fam_mass": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _i64,
                      _i, _f, _p, _p, ctypes.c_size_t, _p]),
    "fam_mass_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fam_compute_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "fam_mass_per_head": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64,
                               _i64, _i, _f, _p, _p, ctypes.c_size_t, _p]),
    "fam_mass_per_head_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fam_kvpop_target": (_i, [_p, _i, _i, _i, _i, _i, _f, _i, _p, _p]),
    "fam_compute": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _i64,
                         _i, _f, _p, _p, _p, ctypes.c_size_t, _p]),
    "evict_plan": (_i, [_i, _i, _p, _i, _i, _p, _p]),
    "fam_budgets_from_ratios": (_i, [_i, _p, _i64, _p]),
    "fam_soft_topk": (_i, [_p, _i, ctypes.c_double, ctypes.c_double, _p]),
    "evict_select": (_i, [_p, _i64, _i, _i, _p, _i, _i, _p, _p, _p, ctypes.c_size_t, _p]),
    "evict_select_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fam_mass_select": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64, _i64,
                             _i, _f, _p, _p, ctypes.c_size_t, _p, _i, _i, _p, _p, _p,
                             ctypes.c_size_t, _p]),
    "evict_select_prepare": (_i, [_p, _i64, _i, _i, _i, _i, _p, ctypes.c_size_t, _p]),
    "evict_select_prepared": (_i, [_p, _i64, _i, _i, _p, _i, _i, _p, _p, _p, ctypes.c_size_t, _p]),
    "fam_mass_prepare_select": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64,
                                     _i64, _i64, _i, _f, _p, _p, ctypes.c_size_t, _i, _i, _p,
                                     ctypes.c_size_t, _p]),
    "evict_select_noalloc": (_i, [_p, _i64, _i, _i, _p, _i, _i, _p, _p, _p]),
    "kv_compact": (_i, [_p, _p, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _p]),
    "fam_compute_chunk": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _i64,
                               _i64, _i, _f, _p, _p, _p, ctypes.c_size_t, _p]),
    "kv_append": (_i, [_p, _p, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _p, _p, _i64, _i64, _i64,
                       _i64, _i, _i, _p, _i64, _i, _p]),
    "kv_compact_inplace": (_i, [_p, _p, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _p, _p, _i64, _p,
                                _i64, _p, ctypes.c_size_t, _p]),
    "kv_compact_inplace_workspace_size": (ctypes.c_size_t, [_i64]),
    "kv_compact_inplace_status": (_i, [_p, _p]),
    "fam_rank_order": (_i, [_p, _i64, _i, _i, _p, _p, ctypes.c_size_t, _p]),
    "fam_rank_order_workspace_size": (ctypes.c_size_t, [_i, _i]),
    "fam_eviction_cost": (_i, [_p, _i64, _p, _i, _i, _p, _p, ctypes.c_size_t, _p]),
    "fam_eviction_cost_workspace_size": (ctypes.c_size_t, [_i, _i]),
    "fam_retention_overlap": (_i, [_p, _p, _p, _p, _i, _i, _p, _p]),
    "fam_eviction_cost_ratio": (_i, [_p, _i64, _p, _i64, _i, _i, _p, _p, ctypes.c_size_t, _p]),
    "fam_eviction_cost_ratio_workspace_size": (ctypes.c_size_t, [_i, _i]),
    "fam_topk_cutoff": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, ctypes.c_size_t, _p]),
    "fam_topk_cutoff_workspace_size": (ctypes.c_size_t, [_i, _i]),
}
EXPORTED = tuple(_SIGNATURES)


class FamError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfam.so once; raise FamError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise FamError(-1, f"{_LIB_PATH} is missing; build it with "
                               "python -m future_attention_scoring_amd.build")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise FamError(status, load().fam_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FAM_BF16
    if t.dtype == torch.float16:
        return FAM_FP16
    raise FamError(2, f"dtype {t.dtype} is not bfloat16 or float16")


def _as4(t: torch.Tensor) -> torch.Tensor:
    if t.dim() == 3:
        return t.unsqueeze(0)
    if t.dim() != 4:
        raise FamError(1, f"expected [B,H,S,d] or [H,S,d], got shape {tuple(t.shape)}")
    return t


def _score_args(q: torch.Tensor, k: torch.Tensor):
    q4, k4 = _as4(q), _as4(k)
    if not (q4.is_cuda and k4.is_cuda):
        raise FamError(1, "q and k must be device tensors")
    if q4.dtype != k4.dtype:
        raise FamError(1, "q and k must share a dtype")
    if q4.stride(3) != 1 or k4.stride(3) != 1:
        raise FamError(1, "the head dimension must be contiguous")
    B, Hq, S, d = q4.shape
    if k4.shape[0] != B or k4.shape[2] != S or k4.shape[3] != d:
        raise FamError(1, f"k shape {tuple(k4.shape)} does not match q {tuple(q4.shape)}")
    Hkv = k4.shape[1]
    return q4, k4, B, Hq, Hkv, S, d


def fam_key_norm_parts(S: int) -> int:
    return int(load().fam_key_norm_parts(int(S)))


def fam_key_norms(k: torch.Tensor, knorm: Optional[torch.Tensor] = None) -> torch.Tensor:
    k4 = _as4(k)
    if not k4.is_cuda or k4.stride(3) != 1:
        raise FamError(1, "k must be a device tensor with a contiguous head dimension")
    B, Hkv, S, d = k4.shape
    P = fam_key_norm_parts(S)
    if knorm is None:
        knorm = torch.empty((B, Hkv, P), dtype=torch.float32, device=k4.device)
    elif knorm.numel() != B * Hkv * P or knorm.dtype != torch.float32 or not knorm.is_contiguous():
        raise FamError(1, f"knorm must be contiguous fp32 [B, Hkv, {P}]")
    _check(load().fam_key_norms(k4.data_ptr(), _dtype_code(k4), B, Hkv, S, d, *k4.stride()[:3],
                                knorm.data_ptr(), _stream(k4)))
    return knorm if k.dim() == 4 else knorm[0]


def fam_lse(q: torch.Tensor, k: torch.Tensor, scale: Optional[float] = None,
            lse: Optional[torch.Tensor] = None, knorm: Optional[torch.Tensor] = None
            ) -> torch.Tensor:
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q4.device)
    kn = 0
    if knorm is not None:
        if (knorm.numel() != B * Hkv * fam_key_norm_parts(S) or knorm.dtype != torch.float32
                or not knorm.is_contiguous()):
            raise FamError(1, "knorm must be fam_key_norms' output for this k")
        kn = knorm.data_ptr()
    _check(load().fam_lse(q4.data_ptr(), k4.data_ptr(), _dtype_code(q4), B, Hq, Hkv, S, d,
                          *q4.stride()[:3], *k4.stride()[:3], 0.0 if scale is None else scale,
                          kn, lse.data_ptr(), _stream(q4)))
    return lse if q.dim() == 4 else lse[0]


def fam_mass_workspace_size(B: int, Hq: int, Hkv: int, S: int) -> int:
    return int(load().fam_mass_workspace_size(int(B), int(Hq), int(Hkv), int(S)))


def _mass_workspace(workspace, B, Hq, Hkv, S, device):
    """The caller's workspace, or one of the recommended size (None if 0)."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    n = fam_mass_workspace_size(B, Hq, Hkv, S)
    if n == 0:
        return None, 0
    # freed on return: torch's allocator reuses it only in stream order
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws.data_ptr(), n


def fam_compute_workspace_size(B: int, Hq: int, Hkv: int, Sq: int, Sk: int) -> int:
    return int(load().fam_compute_workspace_size(int(B), int(Hq), int(Hkv), int(Sq), int(Sk)))


def _compute_workspace(workspace, B, Hq, Hkv, Sq, Sk, device):
    """The caller's workspace, or one of the recommended size for both
    passes of fam_compute / fam_compute_chunk (None if 0)."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    n = fam_compute_workspace_size(B, Hq, Hkv, Sq, Sk)
    if n == 0:
        return None, 0
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws.data_ptr(), n


def fam_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, W: int,
             scale: Optional[float] = None, mass: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    lse = lse.contiguous()
    if lse.numel() != B * Hq * S or lse.dtype != torch.float32:
        raise FamError(1, "lse must be fp32 [B, Hq, S]")
    if mass is None:
        mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=q4.device)
    ws, nbytes = _mass_workspace(workspace, B, Hq, Hkv, S, q4.device)
    _check(load().fam_mass(q4.data_ptr(), k4.data_ptr(), lse.data_ptr(), _dtype_code(q4), B, Hq,
                           Hkv, S, d, *q4.stride()[:3], *k4.stride()[:3], int(W),
                           0.0 if scale is None else scale, mass.data_ptr(), ws, nbytes,
                           _stream(q4)))
    return mass if q.dim() == 4 else mass[0]


def fam_mass_per_head_workspace_size(B: int, Hq: int, Hkv: int, S: int) -> int:
    return int(load().fam_mass_per_head_workspace_size(int(B), int(Hq), int(Hkv), int(S)))


def fam_mass_per_head(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, W: int,
                      scale: Optional[float] = None, mass_q: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-query-head mass [B, Hq, S]. Without a workspace one of
    fam_mass_per_head_workspace_size bytes is allocated (none below 65536
    keys); an empty one runs the pass unsplit."""
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    lse = lse.contiguous()
    if lse.numel() != B * Hq * S or lse.dtype != torch.float32:
        raise FamError(1, "lse must be fp32 [B, Hq, S]")
    if mass_q is None:
        mass_q = torch.empty((B, Hq, S), dtype=torch.float32, device=q4.device)
    if workspace is not None:
        ws, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        nbytes = fam_mass_per_head_workspace_size(B, Hq, Hkv, S)
        # freed on return: torch's allocator reuses it only in stream order
        wt = torch.empty(nbytes, dtype=torch.uint8, device=q4.device) if nbytes else None
        ws = wt.data_ptr() if nbytes else None
    _check(load().fam_mass_per_head(q4.data_ptr(), k4.data_ptr(), lse.data_ptr(), _dtype_code(q4),
                                    B, Hq, Hkv, S, d, *q4.stride()[:3], *k4.stride()[:3], int(W),
                                    0.0 if scale is None else scale, mass_q.data_ptr(), ws, nbytes,
                                    _stream(q4)))
    return mass_q if q.dim() == 4 else mass_q[0]


FAM_AGG = {"max": 0, "mean": 1}


def fam_kvpop_target(mass_q: torch.Tensor, Hkv: int, W: int, eps: float = 0.0,
                     aggregate: str = "max", target: Optional[torch.Tensor] = None
                     ) -> torch.Tensor:
    """KVpop target [B, Hkv, S] (or [Hkv, S]) from per-query-head mass [B, Hq, S]."""
    m = mass_q if mass_q.dim() == 3 else mass_q.unsqueeze(0)
    if m.dim() != 3 or m.dtype != torch.float32 or not m.is_cuda or not m.is_contiguous():
        raise FamError(1, "mass_q must be a contiguous device fp32 [B, Hq, S] tensor")
    if aggregate not in FAM_AGG:
        raise FamError(1, f"aggregate must be one of {sorted(FAM_AGG)}")
    B, Hq, S = m.shape
    if target is None:
        target = torch.empty((B, int(Hkv), S), dtype=torch.float32, device=m.device)
    _check(load().fam_kvpop_target(m.data_ptr(), B, Hq, int(Hkv), S, int(W), float(eps),
                                   FAM_AGG[aggregate], target.data_ptr(), _stream(m)))
    return target if mass_q.dim() == 3 else target[0]


def fam_compute(q: torch.Tensor, k: torch.Tensor, W: int, scale: Optional[float] = None,
                lse: Optional[torch.Tensor] = None, mass: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q4.device)
    if mass is None:
        mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=q4.device)
    ws, nbytes = _compute_workspace(workspace, B, Hq, Hkv, S, S, q4.device)
    _check(load().fam_compute(q4.data_ptr(), k4.data_ptr(), _dtype_code(q4), B, Hq, Hkv, S, d,
                              *q4.stride()[:3], *k4.stride()[:3], int(W),
                              0.0 if scale is None else scale, lse.data_ptr(), mass.data_ptr(),
                              ws, nbytes, _stream(q4)))
    if q.dim() == 3:
        return lse.view(Hq, S), mass.view(Hkv, S)
    return lse, mass


def _i64_array(values: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int64))


def evict_plan(budgets: Sequence[int], S: int, sinks: int, recent: int
               ) -> Tuple[np.ndarray, np.ndarray]:
    b = _i64_array(budgets)
    H = b.size
    kept = np.empty(H, dtype=np.int64)
    offsets = np.empty(H + 1, dtype=np.int64)
    _check(load().evict_plan(H, int(S), b.ctypes.data, int(sinks), int(recent),
                             kept.ctypes.data, offsets.ctypes.data))
    return kept, offsets


def fam_budgets_from_ratios(ratios: Sequence[float], t: int) -> np.ndarray:
    r = np.ascontiguousarray(np.asarray(ratios, dtype=np.float64))
    out = np.empty(r.size, dtype=np.int64)
    _check(load().fam_budgets_from_ratios(r.size, r.ctypes.data, int(t), out.ctypes.data))
    return out


def fam_soft_topk(x: Sequence[float], k: float, tau: float = 1.0) -> np.ndarray:
    """LKV's Soft-TopK masks of x (host, fp64): in (0, 1), summing to k."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64).ravel())
    out = np.empty_like(a)
    _check(load().fam_soft_topk(a.ctypes.data, a.size, float(k), float(tau), out.ctypes.data))
    return out.reshape(np.shape(x))


def evict_select_workspace_size(H: int, S: int, sinks: int, recent: int) -> int:
    return int(load().evict_select_workspace_size(int(H), int(S), int(sinks), int(recent)))


def _select_outputs(scores, budgets, sinks, recent, idx, offsets):
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise FamError(1, "scores must be a device fp32 [H, S] tensor")
    if scores.shape[1] > 1 and scores.stride(1) != 1:
        raise FamError(1, "scores rows must be contiguous")
    H, S = scores.shape
    b = _i64_array(budgets)
    if b.size != H:
        raise FamError(1, f"{b.size} budgets for {H} heads")
    _, host_off = evict_plan(b, S, sinks, recent)
    if idx is None:
        idx = torch.empty(int(host_off[-1]), dtype=torch.int32, device=scores.device)
    if offsets is None:
        offsets = torch.empty(H + 1, dtype=torch.int64, device=scores.device)
    return H, S, b, idx, offsets


def evict_select(scores: torch.Tensor, budgets: Sequence[int], sinks: int, recent: int,
                 idx: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    H, S, b, idx, offsets = _select_outputs(scores, budgets, sinks, recent, idx, offsets)
    if workspace is None:
        nbytes = evict_select_workspace_size(H, S, sinks, recent)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=scores.device)
    _check(load().evict_select(scores.data_ptr(), _row_stride(scores), H, S, b.ctypes.data,
                               int(sinks), int(recent), idx.data_ptr(), offsets.data_ptr(),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream(scores)))
    return idx, offsets


def evict_select_prepare(scores: torch.Tensor, sinks: int, recent: int,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The budget-free first part of evict_select on [H, S] scores, into
    `workspace` (allocated when not given); returns the workspace, which
    evict_select_prepared then takes with any budgets."""
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise FamError(1, "scores must be a device fp32 [H, S] tensor")
    if scores.shape[1] > 1 and scores.stride(1) != 1:
        raise FamError(1, "scores rows must be contiguous")
    H, S = scores.shape
    if workspace is None:
        nbytes = evict_select_workspace_size(H, S, sinks, recent)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=scores.device)
    _check(load().evict_select_prepare(scores.data_ptr(), _row_stride(scores), H, S, int(sinks),
                                       int(recent), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream(scores)))
    return workspace


def evict_select_prepared(scores: torch.Tensor, budgets: Sequence[int], sinks: int, recent: int,
                          workspace: torch.Tensor, idx: Optional[torch.Tensor] = None,
                          offsets: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """evict_select on scores whose workspace evict_select_prepare or
    fam_mass_prepare_select prepared: returns (idx, offsets)."""
    H, S, b, idx, offsets = _select_outputs(scores, budgets, sinks, recent, idx, offsets)
    _check(load().evict_select_prepared(scores.data_ptr(), _row_stride(scores), H, S, b.ctypes.data,
                                        int(sinks), int(recent), idx.data_ptr(), offsets.data_ptr(),
                                        workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(scores)))
    return idx, offsets


def fam_mass_prepare_select(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, W: int, sinks: int,
                            recent: int, scale: Optional[float] = None,
                            mass: Optional[torch.Tensor] = None,
                            mass_workspace: Optional[torch.Tensor] = None,
                            select_workspace: Optional[torch.Tensor] = None
                            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """fam_mass that also prepares evict_select's workspace for its [B * Hkv, S]
    output: returns (mass [B, Hkv, S] (or [Hkv, S]), select_workspace)."""
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    lse = lse.contiguous()
    if lse.numel() != B * Hq * S or lse.dtype != torch.float32:
        raise FamError(1, "lse must be fp32 [B, Hq, S]")
    H = B * Hkv
    if mass is None:
        mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=q4.device)
    if mass_workspace is None:
        n = fam_mass_workspace_size(B, Hq, Hkv, S)
        mass_workspace = torch.empty(n, dtype=torch.uint8, device=q4.device) if n else None
    mws, mbytes = ((mass_workspace.data_ptr(), mass_workspace.numel() * mass_workspace.element_size())
                   if mass_workspace is not None else (None, 0))
    if select_workspace is None:
        nbytes = evict_select_workspace_size(H, S, sinks, recent)
        select_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q4.device)
    _check(load().fam_mass_prepare_select(q4.data_ptr(), k4.data_ptr(), lse.data_ptr(), _dtype_code(q4),
                                          B, Hq, Hkv, S, d, *q4.stride()[:3], *k4.stride()[:3], int(W),
                                          0.0 if scale is None else scale, mass.data_ptr(), mws, mbytes,
                                          int(sinks), int(recent), select_workspace.data_ptr(),
                                          select_workspace.numel() * select_workspace.element_size(),
                                          _stream(q4)))
    return (mass if q.dim() == 4 else mass[0]), select_workspace


def fam_mass_select(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, W: int,
                    budgets: Sequence[int], sinks: int, recent: int, scale: Optional[float] = None,
                    mass: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    offsets: Optional[torch.Tensor] = None,
                    mass_workspace: Optional[torch.Tensor] = None,
                    select_workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """fam_mass and then evict_select on the [B * Hkv, S] masses, in one call:
    returns (mass [B, Hkv, S] (or [Hkv, S]), idx, offsets)."""
    q4, k4, B, Hq, Hkv, S, d = _score_args(q, k)
    lse = lse.contiguous()
    if lse.numel() != B * Hq * S or lse.dtype != torch.float32:
        raise FamError(1, "lse must be fp32 [B, Hq, S]")
    H = B * Hkv
    b = _i64_array(budgets)
    if b.size != H:
        raise FamError(1, f"{b.size} budgets for {H} heads")
    if mass is None:
        mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=q4.device)
    _, host_off = evict_plan(b, S, sinks, recent)
    if idx is None:
        idx = torch.empty(int(host_off[-1]), dtype=torch.int32, device=q4.device)
    if offsets is None:
        offsets = torch.empty(H + 1, dtype=torch.int64, device=q4.device)
    # both workspaces stay referenced until the launches are queued, so that
    # the allocator cannot hand one's memory to the other
    if mass_workspace is None:
        n = fam_mass_workspace_size(B, Hq, Hkv, S)
        mass_workspace = torch.empty(n, dtype=torch.uint8, device=q4.device) if n else None
    mws, mbytes = ((mass_workspace.data_ptr(), mass_workspace.numel() * mass_workspace.element_size())
                   if mass_workspace is not None else (None, 0))
    if select_workspace is None:
        nbytes = evict_select_workspace_size(H, S, sinks, recent)
        select_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q4.device)
    _check(load().fam_mass_select(q4.data_ptr(), k4.data_ptr(), lse.data_ptr(), _dtype_code(q4), B,
                                  Hq, Hkv, S, d, *q4.stride()[:3], *k4.stride()[:3], int(W),
                                  0.0 if scale is None else scale, mass.data_ptr(), mws, mbytes,
                                  b.ctypes.data, int(sinks), int(recent), idx.data_ptr(),
                                  offsets.data_ptr(), select_workspace.data_ptr(),
                                  select_workspace.numel() * select_workspace.element_size(),
                                  _stream(q4)))
    return (mass if q.dim() == 4 else mass[0]), idx, offsets


def evict_select_noalloc(scores: torch.Tensor, budgets: Sequence[int], sinks: int, recent: int,
                         idx: torch.Tensor, offsets: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """evict_select with the library's static scratch instead of a workspace;
    the caller passes idx [offsets[H]] int32 and offsets [H + 1] int64."""
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise FamError(1, "scores must be a device fp32 [H, S] tensor")
    if scores.shape[1] > 1 and scores.stride(1) != 1:
        raise FamError(1, "scores rows must be contiguous")
    H, S = scores.shape
    b = _i64_array(budgets)
    if b.size != H:
        raise FamError(1, f"{b.size} budgets for {H} heads")
    _check(load().evict_select_noalloc(scores.data_ptr(), _row_stride(scores), H, S, b.ctypes.data,
                                       int(sinks), int(recent), idx.data_ptr(), offsets.data_ptr(),
                                       _stream(scores)))
    return idx, offsets


def kv_compact(k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, offsets: torch.Tensor,
               total_rows: Optional[int] = None, k_new: Optional[torch.Tensor] = None,
               v_new: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    if k.dim() != 3 or v.shape != k.shape or k.dtype != v.dtype:
        raise FamError(1, "k and v must be [H, S, d] tensors of one dtype and shape")
    if k.element_size() != 2 or k.stride(2) != 1 or v.stride(2) != 1:
        raise FamError(1, "k and v need 2-byte elements with a contiguous last axis")
    H, S, d = k.shape
    rows = int(idx.numel()) if total_rows is None else int(total_rows)
    if k_new is None:
        k_new = torch.empty((rows, d), dtype=k.dtype, device=k.device)
    if v_new is None:
        v_new = torch.empty((rows, d), dtype=v.dtype, device=v.device)
    _check(load().kv_compact(k.data_ptr(), v.data_ptr(), 2, H, S, d, k.stride(0), k.stride(1),
                             v.stride(0), v.stride(1), idx.data_ptr(), offsets.data_ptr(), rows,
                             k_new.data_ptr(), v_new.data_ptr(), _stream(k)))
    return k_new, v_new


def fam_compute_chunk(q: torch.Tensor, k: torch.Tensor, W: int, scale: Optional[float] = None,
                      lse: Optional[torch.Tensor] = None, mass: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Scores of a chunk's Sq queries over Sk cache rows (the chunk's own keys
    last): lse [B, Hq, Sq] and mass [B, Hkv, Sk] (3-D inputs give 2-D outputs)."""
    q4, k4 = _as4(q), _as4(k)
    if not (q4.is_cuda and k4.is_cuda) or q4.dtype != k4.dtype:
        raise FamError(1, "q and k must be device tensors of one dtype")
    if q4.stride(3) != 1 or k4.stride(3) != 1:
        raise FamError(1, "the head dimension must be contiguous")
    B, Hq, Sq, d = q4.shape
    if k4.shape[0] != B or k4.shape[3] != d:
        raise FamError(1, f"k shape {tuple(k4.shape)} does not match q {tuple(q4.shape)}")
    Hkv, Sk = k4.shape[1], k4.shape[2]
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q4.device)
    if mass is None:
        mass = torch.empty((B, Hkv, Sk), dtype=torch.float32, device=q4.device)
    ws, nbytes = _compute_workspace(workspace, B, Hq, Hkv, Sq, Sk, q4.device)
    _check(load().fam_compute_chunk(q4.data_ptr(), k4.data_ptr(), _dtype_code(q4), B, Hq, Hkv,
                                    Sq, Sk, d, *q4.stride()[:3], *k4.stride()[:3], int(W),
                                    0.0 if scale is None else scale, lse.data_ptr(),
                                    mass.data_ptr(), ws, nbytes, _stream(q4)))
    if q.dim() == 3:
        return lse.view(Hq, Sq), mass.view(Hkv, Sk)
    return lse, mass


def _cache_args(k: torch.Tensor, v: torch.Tensor, what: str):
    if k.dim() != 3 or v.dim() != 3 or k.shape != v.shape or k.dtype != v.dtype:
        raise FamError(1, f"{what}: k and v must be [H, rows, d] tensors of one shape and dtype")
    if k.element_size() != 2 or k.stride(2) != 1 or v.stride(2) != 1 or not k.is_cuda:
        raise FamError(1, f"{what}: device tensors with 2-byte elements and a contiguous last axis")
    return k.shape


def kv_append(k_src: torch.Tensor, v_src: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, row0: int, pos: Optional[torch.Tensor] = None,
              pos0: int = 0) -> None:
    """Copy [H, n, d] rows into cache rows row0 .. row0+n-1 (and their positions)."""
    H, n, d = _cache_args(k_src, v_src, "kv_append source")
    Hc, cap, dc = _cache_args(k_cache, v_cache, "kv_append cache")
    if Hc != H or dc != d:
        raise FamError(1, f"cache {tuple(k_cache.shape)} does not match rows {tuple(k_src.shape)}")
    pp, psh = 0, 0
    if pos is not None:
        if (pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[0] != H or pos.shape[1] < cap
                or pos.stride(1) != 1 or not pos.is_cuda):
            raise FamError(1, "pos must be a device int32 [H, capacity] with contiguous rows")
        pp, psh = pos.data_ptr(), pos.stride(0)
    _check(load().kv_append(k_src.data_ptr(), v_src.data_ptr(), 2, H, n, d, k_src.stride(0),
                            k_src.stride(1), v_src.stride(0), v_src.stride(1), k_cache.data_ptr(),
                            v_cache.data_ptr(), k_cache.stride(0), k_cache.stride(1),
                            v_cache.stride(0), v_cache.stride(1), cap, int(row0), pp, psh,
                            int(pos0), _stream(k_cache)))


def kv_compact_inplace_workspace_size(total_rows: int) -> int:
    return int(load().kv_compact_inplace_workspace_size(int(total_rows)))


def kv_compact_inplace_status(workspace: torch.Tensor) -> None:
    """Wait for the current stream and raise FamError(FAM_ERR_TIMEOUT) if the
    last kv_compact_inplace on `workspace` left rows unwritten."""
    _check(load().kv_compact_inplace_status(workspace.data_ptr(), _stream(workspace)))


def kv_compact_inplace(k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor,
                       offsets: torch.Tensor, pos: Optional[torch.Tensor] = None,
                       total_rows: Optional[int] = None,
                       workspace: Optional[torch.Tensor] = None) -> None:
    """Move each head's rows idx[offsets[h]:offsets[h+1]] to its first rows
    (total_rows = offsets[H], idx.numel() by default)."""
    H, S, d = _cache_args(k_cache, v_cache, "kv_compact_inplace")
    total = int(idx.numel()) if total_rows is None else int(total_rows)
    if workspace is None:
        workspace = torch.empty(max(kv_compact_inplace_workspace_size(total), 4), dtype=torch.uint8,
                                device=k_cache.device)
    if idx.dtype != torch.int32 or offsets.dtype != torch.int64 or offsets.numel() != H + 1:
        raise FamError(1, "idx must be int32 and offsets int64 [H + 1]")
    pp, psh = 0, 0
    if pos is not None:
        if (pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[0] != H or pos.shape[1] < S
                or pos.stride(1) != 1 or not pos.is_cuda):
            raise FamError(1, "pos must be a device int32 [H, S] with contiguous rows")
        pp, psh = pos.data_ptr(), pos.stride(0)
    _check(load().kv_compact_inplace(k_cache.data_ptr(), v_cache.data_ptr(), 2, H, S, d,
                                     k_cache.stride(0), k_cache.stride(1), v_cache.stride(0),
                                     v_cache.stride(1), idx.data_ptr(), offsets.data_ptr(),
                                     total, pp, psh, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(k_cache)))


class ChunkedCache:
    """A static per-head cache driven by chunked prefill and compression.

    KVP (section 4: long contexts are prefilled chunk by chunk and the cache
    is compressed to the budget after each chunk, with physical compaction)
    and the pruning blog (conclusion: a static cache keeps a fixed region per
    head and overwrites old entries in place). Each chunk is appended after
    the rows the cache holds, scored by the future-attention mass its own
    queries give every cache row (with the normalisers of the attention over
    the cache, i.e. over the retained keys), and then, if the cache exceeds
    the budget, the best-scored rows are kept (sinks and the recent window
    forced, ties to the earlier position) and compacted in place. The budget
    is uniform over heads (a total per head, forced rows included), so every
    head holds the same number of rows. All device work runs in libfam.
    """

    def __init__(self, B: int, Hq: int, Hkv: int, d: int, chunk: int, budget: int, sinks: int,
                 window: int, dtype=torch.bfloat16, device="cuda", scale: Optional[float] = None):
        if min(B, Hq, Hkv, d, chunk) < 1 or budget < 0 or sinks < 0 or window < 0:
            raise FamError(1, "invalid cache sizes")
        self.B, self.Hq, self.Hkv, self.d = B, Hq, Hkv, d
        self.chunk, self.budget, self.sinks, self.window = chunk, budget, sinks, window
        self.scale = scale
        self.capacity = max(budget, sinks + window) + chunk
        H = B * Hkv
        self.k = torch.empty((H, self.capacity, d), dtype=dtype, device=device)
        self.v = torch.empty_like(self.k)
        self.pos = torch.full((H, self.capacity), -1, dtype=torch.int32, device=device)
        self.compact_ws = torch.empty(kv_compact_inplace_workspace_size(H * self.capacity),
                                      dtype=torch.uint8, device=device)
        self.n = 0          # rows held per head
        self.next_pos = 0   # position of the next appended row
        self.lse = None
        self.mass = None

    def append(self, k_chunk: torch.Tensor, v_chunk: torch.Tensor) -> None:
        """k_chunk, v_chunk: [B, Hkv, n, d] (or [B*Hkv, n, d]), n <= chunk."""
        kc = k_chunk.reshape(-1, *k_chunk.shape[-2:])
        vc = v_chunk.reshape(-1, *v_chunk.shape[-2:])
        n = kc.shape[1]
        if n > self.chunk:
            raise FamError(1, f"{n} rows exceed the chunk size {self.chunk}")
        kv_append(kc, vc, self.k, self.v, self.n, self.pos, self.next_pos)
        self.n += n
        self.next_pos += n

    def score(self, q_chunk: torch.Tensor, workspace: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
        """Normalisers [B, Hq, Sq] of the chunk's queries (the last Sq appended
        positions) and the mass [B, Hkv, n] of every cache row."""
        k = self.k[:, :self.n].view(self.B, self.Hkv, self.n, self.d)
        self.lse, self.mass = fam_compute_chunk(q_chunk, k, self.window, self.scale,
                                                workspace=workspace)
        return self.lse, self.mass

    def select(self) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
        """Rows each head keeps by the last mass (evict_select): (idx, offsets),
        or (None, None) if the cache is within the budget."""
        if self.n <= self.budget:
            return None, None
        H = self.B * self.Hkv
        return evict_select(self.mass.view(H, self.n), [self.budget] * H, self.sinks, self.window)

    def compact(self, idx: torch.Tensor, offsets: torch.Tensor) -> None:
        """Move the kept rows to the front of every head's region, in place."""
        kv_compact_inplace(self.k, self.v, idx, offsets, self.pos, workspace=self.compact_ws)
        self.n = int(idx.numel()) // (self.B * self.Hkv)

    def compress(self) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
        """select() then compact(); returns (idx, offsets) or (None, None)."""
        idx, offsets = self.select()
        if idx is not None:
            self.compact(idx, offsets)
        return idx, offsets


def prefill_compress(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunk: int, budget: int,
                     sinks: int, window: int, scale: Optional[float] = None) -> ChunkedCache:
    """Chunked prefill with compression after every chunk over q [B, Hq, S, d],
    k, v [B, Hkv, S, d]; returns the final cache (rows, positions, count)."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    cache = ChunkedCache(B, Hq, Hkv, d, chunk, budget, sinks, window, k.dtype, k.device, scale)
    ws = None
    for p0 in range(0, S, chunk):
        p1 = min(S, p0 + chunk)
        cache.append(k[:, :, p0:p1], v[:, :, p0:p1])
        need = fam_compute_workspace_size(B, Hq, Hkv, p1 - p0, cache.n)
        if ws is None or ws.numel() < need:
            n = max(need, fam_compute_workspace_size(B, Hq, Hkv, p1 - p0, cache.capacity))
            ws = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
        cache.score(q[:, :, p0:p1], workspace=ws)
        cache.compress()
    return cache


def _score_rows(x: torch.Tensor, what: str) -> Tuple[int, int]:
    if x.dim() != 2 or x.dtype != torch.float32 or not x.is_cuda or (x.shape[1] > 1 and x.stride(1) != 1):
        raise FamError(1, f"{what} must be a device fp32 [H, n] tensor with contiguous rows")
    return x.shape[0], x.shape[1]


def _row_stride(x: torch.Tensor) -> int:
    """Row stride of a 2-D tensor; a single row's stride is irrelevant (torch
    may report any value for a dimension of size 1)."""
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def fam_rank_order_workspace_size(H: int, n: int) -> int:
    return int(load().fam_rank_order_workspace_size(int(H), int(n)))


def fam_rank_order(scores: torch.Tensor, order: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Positions of each row's entries, best first (ties to the lower position)."""
    H, n = _score_rows(scores, "scores")
    if order is None:
        order = torch.empty((H, n), dtype=torch.int32, device=scores.device)
    if workspace is None:
        workspace = torch.empty(max(fam_rank_order_workspace_size(H, n), 8), dtype=torch.uint8,
                                device=scores.device)
    _check(load().fam_rank_order(scores.data_ptr(), _row_stride(scores), H, n, order.data_ptr(),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(scores)))
    return order


def fam_eviction_cost_workspace_size(H: int, n: int) -> int:
    return int(load().fam_eviction_cost_workspace_size(int(H), int(n)))


def fam_eviction_cost(importance: torch.Tensor, order: torch.Tensor,
                      cost: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Importance evicted by `order`, summed over all budgets: [H] fp64."""
    H, n = _score_rows(importance, "importance")
    if order.dtype != torch.int32 or tuple(order.shape) != (H, n) or not order.is_contiguous():
        raise FamError(1, "order must be a contiguous int32 [H, n] tensor")
    if cost is None:
        cost = torch.empty(H, dtype=torch.float64, device=importance.device)
    if workspace is None:
        workspace = torch.empty(max(fam_eviction_cost_workspace_size(H, n), 8), dtype=torch.uint8,
                                device=importance.device)
    _check(load().fam_eviction_cost(importance.data_ptr(), _row_stride(importance), order.data_ptr(), H,
                                    n, cost.data_ptr(), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(importance)))
    return cost


def fam_eviction_cost_ratio_workspace_size(H: int, n: int) -> int:
    return int(load().fam_eviction_cost_ratio_workspace_size(int(H), int(n)))


def fam_eviction_cost_ratio(scores: torch.Tensor, importance: torch.Tensor,
                            ratio: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """KVP's normalised eviction cost of ranking by `scores`: cost over the cost
    of ranking by `importance` itself (>= 1; 1 is optimal), per row: [H] fp64."""
    H, n = _score_rows(scores, "scores")
    if _score_rows(importance, "importance") != (H, n):
        raise FamError(1, "scores and importance must have the same [H, n] shape")
    if ratio is None:
        ratio = torch.empty(H, dtype=torch.float64, device=scores.device)
    if workspace is None:
        workspace = torch.empty(max(fam_eviction_cost_ratio_workspace_size(H, n), 8), dtype=torch.uint8,
                                device=scores.device)
    _check(load().fam_eviction_cost_ratio(scores.data_ptr(), _row_stride(scores), importance.data_ptr(),
                                          _row_stride(importance), H, n, ratio.data_ptr(),
                                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                          _stream(scores)))
    return ratio


eviction_cost_ratio = fam_eviction_cost_ratio


def fam_retention_overlap(idx_a: torch.Tensor, offsets_a: torch.Tensor, idx_b: torch.Tensor,
                          offsets_b: torch.Tensor, S: int,
                          common: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per head, the number of positions both kept lists hold: [H] int64."""
    H = offsets_a.numel() - 1
    if offsets_b.numel() != H + 1 or offsets_a.dtype != torch.int64 or offsets_b.dtype != torch.int64:
        raise FamError(1, "offsets must be int64 [H + 1] tensors of one length")
    if idx_a.dtype != torch.int32 or idx_b.dtype != torch.int32:
        raise FamError(1, "idx lists must be int32")
    if common is None:
        common = torch.empty(H, dtype=torch.int64, device=idx_a.device)
    _check(load().fam_retention_overlap(idx_a.data_ptr(), offsets_a.data_ptr(), idx_b.data_ptr(),
                                        offsets_b.data_ptr(), H, int(S), common.data_ptr(),
                                        _stream(idx_a)))
    return common


def fam_topk_cutoff_workspace_size(H: int, S: int) -> int:
    return int(load().fam_topk_cutoff_workspace_size(int(H), int(S)))


def fam_topk_cutoff(order: torch.Tensor, sinks: int, w: int, k: int, tau: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """KVpop's running cut-off tau [H, S] (Algorithm 2, budget (sinks, w, k))
    from fam_rank_order's order [H, S]; -1 where fewer than k are eligible."""
    if order.dim() != 2 or order.dtype != torch.int32 or not order.is_cuda or not order.is_contiguous():
        raise FamError(1, "order must be a contiguous device int32 [H, S] tensor")
    H, S = order.shape
    if tau is None:
        tau = torch.empty((H, S), dtype=torch.int32, device=order.device)
    if workspace is None:
        workspace = torch.empty(max(fam_topk_cutoff_workspace_size(H, S), 4), dtype=torch.uint8,
                                device=order.device)
    _check(load().fam_topk_cutoff(order.data_ptr(), H, S, int(sinks), int(w), int(k), tau.data_ptr(),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(order)))
    return tau
