"""Benchmark of the future-attention-mass + eviction hot path on one MI355X.

One step = fam_key_norms + fam_lse (first pass, bounded form) + fam_mass
(the key-major second pass) +
evict_select (per-head budgets b_h = floor(r_h * S), 4 sinks, recent window)
+ kv_compact (gather of the kept K/V rows), on the Llama-3.1-8B-like layer at
128k tokens (32 query / 8 KV heads, d = 128, bf16, W = 512). Inputs are
seeded synthetic tensors, resident in HBM before timing starts.

Prints one JSON line. `value` is causal key-query pairs per second of the
whole step; `roofline` describes the slowest kernel (algorithmic work per
launch over its mean HIP-event duration); `cpu_baseline` times the fp64
oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--target-steps N] [--ranking-runs N]
                       [--chunked-runs N]

Three widened rows are timed apart from the step and reported beside it:
the KVpop target (per-query-head mass and its epilogue), the ranking-quality
measures (order, eviction cost over budgets, retention overlap) on the
step's masses, and the chunked prefill-compress loop (chunks of 4096, a
uniform budget of 16384 rows per head, compaction in place).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np
import torch

from future_attention_scoring_amd import fam, workloads

PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA (published)
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E (published)
WORKLOADS = {
    "llama-128k": workloads.llama31_8b_128k,
    "qwen3-4b-8k": workloads.qwen3_4b_layer,
    "long-trace-32k": workloads.long_trace,
}


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {
    "fam_lse": ["fam_lse.hip", "fam_device.hpp", "fam_kernels.hpp"],
    "fam_mass": ["fam_mass.hip", "fam_device.hpp", "fam_kernels.hpp"],
    "evict_select": ["evict_select.hip", "fam_device.hpp", "fam_kernels.hpp"],
    "kv_compact": ["kv_compact.hip", "fam_device.hpp", "fam_kernels.hpp"],
    "fam_mass_per_head": ["fam_mass.hip", "fam_device.hpp", "fam_kernels.hpp"],
    "fam_kvpop_target": ["kvpop_target.hip", "fam_device.hpp", "fam_kernels.hpp"],
}


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "future_attention_scoring_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary.

    A kernel's figure is used only if its source hash still matches the one
    recorded with the counters; otherwise it is None.
    """
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] in KERNEL_SOURCES:
                if source_hash(parts[1]) == parts[2]:
                    out[parts[1]] = float(parts[3])
    return out


def algorithmic_work(wl, kept_total):
    """Counts the bench divides by (per launch)."""
    S, W, Hq, Hkv, d = wl.S, wl.W, wl.Hq, wl.Hkv, wl.d
    causal_pairs = Hq * S * (S + 1) // 2
    future_pairs = Hq * (S - W) * (S - W + 1) // 2 if W < S else 0
    esize = 2
    return {
        "causal_pairs": causal_pairs,
        "lse_flops": 2 * d * causal_pairs,
        "mass_flops": 2 * d * future_pairs,
        "select_bytes": 4 * Hkv * S + 4 * kept_total,
        "compact_bytes": 2 * 2 * kept_total * d * esize,
    }


def cpu_baseline(wl, prefix=32768):
    """Time the fp64 oracle on the first `prefix` positions of KV group 0."""
    from oracle import fam_oracle  # test infrastructure: only this leg uses it
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    g = wl.group
    q = wl.q_heads(range(g))[:, :prefix].astype(np.float32)
    k = wl.k_heads([0])[:, :prefix].astype(np.float32)
    q64 = workloads.to_dtype(q, wl.dtype).to(torch.float64).numpy()
    k64 = workloads.to_dtype(k, wl.dtype).to(torch.float64).numpy()
    t0 = time.perf_counter()
    fam_oracle.fam(q64, k64, wl.W)
    dt = time.perf_counter() - t0
    pairs = g * prefix * (prefix + 1) // 2
    return {"value": pairs / dt, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": (f"oracle LSE + mass (fp64) on the first {prefix} positions of KV group 0 "
                       f"({g} query heads) of {wl.name}; {pairs} causal pairs")}


def oracle_select_compact(wl, host, with_decode):
    """The oracle's select (lexsort) + compact (fancy-index gather of K and V)
    timed on the host: on the headline workload's masses and K/V, and on
    every cell of the decode-time sweep (the cells' K/V drawn on the device
    as the sweep draws them, copied to the host)."""
    from oracle import select_oracle  # test infrastructure: only this leg uses it
    out = {}
    t0 = time.perf_counter()
    idx, off = select_oracle.select(host["mass"], host["budgets"], wl.sinks, wl.recent)
    t1 = time.perf_counter()
    select_oracle.compact(host["k"], idx, off)
    select_oracle.compact(host["v"], idx, off)
    t2 = time.perf_counter()
    nbytes = 4 * wl.Hkv * wl.S + 4 * int(off[-1]) + 2 * 2 * int(off[-1]) * wl.d * 2
    out[wl.name] = {"select_s": round(t1 - t0, 4), "compact_s": round(t2 - t1, 4), "bytes": nbytes,
                    "GBps": round(nbytes / (t2 - t0) / 1e9, 3)}
    if with_decode:
        cells = workloads.decode_sweep()
        dev = torch.device("cuda:0")
        rows = []
        for S in workloads.DECODE_CONTEXTS:
            first = [c for c in cells if c.S == S][0]
            gen = torch.Generator(device=dev).manual_seed(first.seed * 1000003 + S)
            kd = torch.randn((first.H, S, first.d), generator=gen, device=dev, dtype=torch.float32).to(first.dtype)
            vd = torch.randn((first.H, S, first.d), generator=gen, device=dev, dtype=torch.float32).to(first.dtype)
            kh, vh = kd.cpu().view(torch.int16).numpy(), vd.cpu().view(torch.int16).numpy()
            del kd, vd
            scores = first.scores()
            for cell in [c for c in cells if c.S == S]:
                budgets = [cell.budget] * cell.H
                t0 = time.perf_counter()
                idx, off = select_oracle.select(scores, budgets, cell.sinks, cell.recent)
                t1 = time.perf_counter()
                select_oracle.compact(kh, idx, off)
                select_oracle.compact(vh, idx, off)
                t2 = time.perf_counter()
                nbytes = 4 * cell.H * S + 4 * int(off[-1]) + 2 * 2 * int(off[-1]) * cell.d * 2
                rows.append({"S": S, "budget": cell.budget, "select_s": round(t1 - t0, 4),
                             "compact_s": round(t2 - t1, 4), "GBps": round(nbytes / (t2 - t0) / 1e9, 3)})
            del kh, vh
        out["decode_sweep"] = rows
    return out


def kvpop_target_row(steps, q, k, lse, wl, work, stream):
    """Time the widened row apart from the step: per-query-head mass (the
    second pass writing [B, Hq, S]) and the KVpop epilogue (count
    normalisation, log, max over the group)."""
    B, Hq, Hkv, S = 1, wl.Hq, wl.Hkv, wl.S
    mass_q = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    target = torch.empty((B, Hkv, S), dtype=torch.float32, device=q.device)
    mq_ws = torch.empty(fam.fam_mass_per_head_workspace_size(B, Hq, Hkv, S), dtype=torch.uint8, device=q.device)

    def run(e=None):
        if e:
            e[0].record(stream)
        fam.fam_mass_per_head(q, k, lse, wl.W, mass_q=mass_q, workspace=mq_ws)
        if e:
            e[1].record(stream)
        fam.fam_kvpop_target(mass_q, Hkv, wl.W, eps=0.0, aggregate="max", target=target)
        if e:
            e[2].record(stream)

    run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        run(e)
    torch.cuda.synchronize()
    mq_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    tg_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    tg_bytes = 4 * B * Hq * S + 4 * B * Hkv * S
    mq_flops = work["mass_flops"] / (mq_ms * 1e-3)
    tg_bw = tg_bytes / (tg_ms * 1e-3)
    return {
        "fam_mass_per_head": {"bound": "mfma", "achieved": round(mq_flops / 1e12, 3),
                              "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                              "frac": round(mq_flops / PEAK_BF16_FLOPS, 4), "ms": round(mq_ms, 4)},
        "fam_kvpop_target": {"bound": "hbm", "achieved": round(tg_bw / 1e9, 3),
                             "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                             "frac": round(tg_bw / PEAK_HBM_BYTES, 4), "ms": round(tg_ms, 4),
                             "bytes": tg_bytes},
        "steps": steps,
    }


def chunked_row(runs, q, k, v, wl, stream, chunk=4096, budget=16384):
    """Time the chunked prefill-compress loop over the whole sequence apart
    from the step: per chunk, kv_append of its K/V rows, fam_compute_chunk
    (key norms, first pass and mass of the chunk's queries over the cache),
    and, once the cache exceeds the budget, evict_select + in-place
    compaction (ChunkedCache.compress). The budget is uniform per head."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    cap = max(budget, wl.sinks + wl.W) + chunk
    ws_n = max([fam.fam_compute_workspace_size(B, Hq, Hkv, chunk, s) for s in range(chunk, cap + 1, chunk)] + [16])
    ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device)

    def one(record):
        cache = fam.ChunkedCache(B, Hq, Hkv, d, chunk, budget, wl.sinks, wl.W, k.dtype, q.device)
        marks, sizes, moved = [], [], []
        for p0 in range(0, S, chunk):
            p1 = min(S, p0 + chunk)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
            if e:
                e[0].record(stream)
            n_old = cache.n
            cache.append(k[:, :, p0:p1], v[:, :, p0:p1])
            if e:
                e[1].record(stream)
            cache.score(q[:, :, p0:p1], workspace=ws)
            if e:
                e[2].record(stream)
            idx, offsets = cache.select()
            if e:
                e[3].record(stream)
            if idx is not None:
                if not record:   # rows that move (idx[r] != r), counted in the untimed run only
                    rows = torch.arange(idx.numel() // (B * Hkv), device=idx.device, dtype=idx.dtype)
                    moved.append(int((idx.view(B * Hkv, -1) != rows).sum()))
                cache.compact(idx, offsets)
            if e:
                e[4].record(stream)
            marks.append(e)
            sizes.append((n_old, p1 - p0))
        return marks, sizes, moved

    _, _, moved = one(False)
    torch.cuda.synchronize()
    per_run = []
    for _ in range(runs):
        t0 = time.perf_counter()
        marks, sizes, _ = one(True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        phases = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in marks]).sum(axis=0)
        per_run.append((wall * 1e3, phases))
    wall_ms = float(np.mean([r[0] for r in per_run]))
    append_ms, score_ms, select_ms, compact_ms = (float(x) for x in np.mean([r[1] for r in per_run], axis=0))
    compact_bytes = 2 * 2 * sum(moved) * d * k.element_size()   # K and V rows, read + write
    W = wl.W
    lse_pairs = sum(Hq * (c * n + c * (c + 1) // 2) for n, c in sizes)
    mass_pairs = sum(Hq * sum(max(0, n + i - W + 1) for i in range(c)) for n, c in sizes)
    flops = 2 * d * (lse_pairs + mass_pairs)
    return {
        "workload": f"{wl.name} chunked prefill-compress",
        "chunk": chunk, "budget_per_head": budget, "sinks": wl.sinks, "window": W,
        "chunks": len(sizes), "runs": runs,
        "pairs_per_s": lse_pairs / (wall_ms * 1e-3),
        "causal_pairs": lse_pairs, "future_pairs": mass_pairs,
        "ms_wall": round(wall_ms, 3),
        "ms": {"kv_append": round(append_ms, 3), "fam_compute_chunk": round(score_ms, 3),
               "evict_select": round(select_ms, 3), "kv_compact_inplace": round(compact_ms, 3)},
        "fam_compute_chunk": {"bound": "mfma", "achieved": round(flops / (score_ms * 1e-3) / 1e12, 3),
                              "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                              "frac": round(flops / (score_ms * 1e-3) / PEAK_BF16_FLOPS, 4)},
        "kv_compact_inplace": {"bound": "hbm", "moved_rows": int(sum(moved)), "bytes": compact_bytes,
                               "achieved": round(compact_bytes / (compact_ms * 1e-3) / 1e9, 3),
                               "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                               "frac": round(compact_bytes / (compact_ms * 1e-3) / PEAK_HBM_BYTES, 4)},
    }


def ranking_row(runs, mass, wl, stream):
    """Time the ranking-quality row on the step's masses: fam_rank_order of the
    masses (the teacher's order) and of a recency score (newest first),
    fam_eviction_cost of both against the masses (KVP's cost over budgets and
    its normalised form), fam_retention_overlap of the two kept sets at a
    budget of S/8 (KVpop's top-k retention recall), and fam_topk_cutoff of the
    mass order (KVpop's running cut-off, the workload's sinks, window W,
    k = S/8)."""
    m = mass[0]
    H, S = m.shape
    recency = torch.arange(S, dtype=torch.float32, device=m.device).expand(H, S).contiguous()
    order = torch.empty((H, S), dtype=torch.int32, device=m.device)
    ws = torch.empty(max(8, fam.fam_rank_order_workspace_size(H, S)), dtype=torch.uint8, device=m.device)
    cost = torch.empty(H, dtype=torch.float64, device=m.device)
    cost_ws = torch.empty(max(8, fam.fam_eviction_cost_workspace_size(H, S)), dtype=torch.uint8, device=m.device)
    budgets = [S // 8] * H
    ia, oa = fam.evict_select(m, budgets, wl.sinks, wl.recent)
    ib, ob = fam.evict_select(recency, budgets, wl.sinks, wl.recent)

    tau = torch.empty((H, S), dtype=torch.int32, device=m.device)
    cut_ws = torch.empty(max(4, fam.fam_topk_cutoff_workspace_size(H, S)), dtype=torch.uint8, device=m.device)

    def one(e=None):
        if e:
            e[0].record(stream)
        fam.fam_rank_order(m, order=order, workspace=ws)
        if e:
            e[1].record(stream)
        fam.fam_eviction_cost(m, order, cost=cost, workspace=cost_ws)
        if e:
            e[2].record(stream)
        common = fam.fam_retention_overlap(ia, oa, ib, ob, S)
        if e:
            e[3].record(stream)
        fam.fam_topk_cutoff(order, wl.sinks, wl.W, S // 8, tau=tau, workspace=cut_ws)
        if e:
            e[4].record(stream)
        return common

    one()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(runs)]
    for e in ev:
        common = one(e)
    torch.cuda.synchronize()
    ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev])) for i in range(4)]
    ratio = fam.eviction_cost_ratio(recency, m).cpu().numpy()
    recall = (common.double() / (oa[1:] - oa[:-1]).double()).cpu().numpy()
    rank_bytes = 2 * 4 * H * S   # scores in, order out
    return {
        "heads": H, "entries_per_head": S, "runs": runs,
        "ms": {"fam_rank_order": round(ms[0], 4), "fam_eviction_cost": round(ms[1], 4),
               "fam_retention_overlap": round(ms[2], 4), "fam_topk_cutoff": round(ms[3], 4)},
        "fam_topk_cutoff": {"sinks": wl.sinks, "window": wl.W, "k": S // 8, "queries_per_head": S,
                            "queries_per_s": round(H * S / (ms[3] * 1e-3), 1)},
        "fam_rank_order": {"bound": "latency", "bytes": rank_bytes,
                           "achieved": round(rank_bytes / (ms[0] * 1e-3) / 1e9, 3), "unit": "GB/s",
                           "note": ("four stable radix passes; up to 64 tiles of 4096 a head (this row) each is two launches "
                                    "(tile counts, place), beyond that three (counts, per-head scan, place)")},
        "recency_vs_mass": {"normalised_cost_mean": round(float(ratio.mean()), 6),
                            "retention_recall_mean_at_S_over_8": round(float(recall.mean()), 6)},
    }


def decode_row(runs, stream):
    """Time the decode-time eviction sweep apart from the step: a
    Qwen2.5-1.5B-like cache (28 layers x 2 KV heads = 56 slices, d = 128,
    fp16 K/V), given fp32 scores ~ Exp(1), 4 sinks + 32 recent + the best of
    the rest to budgets {4096, 2048, 1024, 512} at contexts {512, 4096,
    32768, 120000}: evict_select + kv_compact into a new cache per cell.
    K/V are seeded normal values drawn on the device (only their size
    matters for the timing); the scores come from the same seeded generator
    as the parity tests. Before every run a 512 MiB fill (outside the timed
    events) evicts the L2s and the 256 MB MALL, so that the repeated runs
    read their scores and K/V rows from HBM."""
    dev = torch.device("cuda:0")
    cells = workloads.decode_sweep()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    rows, tot_bytes, tot_us = [], 0, 0.0
    for S in workloads.DECODE_CONTEXTS:
        first = [c for c in cells if c.S == S][0]
        H, d = first.H, first.d
        gen = torch.Generator(device=dev).manual_seed(first.seed * 1000003 + S)
        k = torch.randn((H, S, d), generator=gen, device=dev, dtype=torch.float32).to(first.dtype)
        v = torch.randn((H, S, d), generator=gen, device=dev, dtype=torch.float32).to(first.dtype)
        scores = torch.from_numpy(first.scores()).to(dev)
        for cell in [c for c in cells if c.S == S]:
            budgets = [cell.budget] * H
            _, off = fam.evict_plan(budgets, S, cell.sinks, cell.recent)
            total = int(off[-1])
            idx = torch.empty(total, dtype=torch.int32, device=dev)
            offd = torch.empty(H + 1, dtype=torch.int64, device=dev)
            ws = torch.empty(max(16, fam.evict_select_workspace_size(H, S, cell.sinks, cell.recent)),
                             dtype=torch.uint8, device=dev)
            kn = torch.empty((total, d), dtype=k.dtype, device=dev)
            vn = torch.empty_like(kn)

            def run(e=None):
                if e:
                    e[0].record(stream)
                fam.evict_select(scores, budgets, cell.sinks, cell.recent, idx=idx, offsets=offd, workspace=ws)
                if e:
                    e[1].record(stream)
                fam.kv_compact(k, v, idx, offd, total, k_new=kn, v_new=vn)
                if e:
                    e[2].record(stream)

            for _ in range(2):
                flush.fill_(0)
                run()
            torch.cuda.synchronize()
            # all timed runs enqueued before one synchronisation, so that the
            # host's per-call work overlaps the GPU's and the events time the
            # GPU alone
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(runs)]
            for i, e in enumerate(evs):
                flush.fill_(i & 0x7f)
                run(e)
            torch.cuda.synchronize()
            sel = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
            cmp_ = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
            s_us, c_us = float(np.median(sel)), float(np.median(cmp_))
            # scores read, indices written, kept K and V rows read and written
            nbytes = 4 * H * S + 4 * total + 2 * 2 * total * d * k.element_size()
            tot_bytes += nbytes
            tot_us += s_us + c_us
            rows.append({"S": S, "budget": cell.budget, "kept_rows": total, "select_us": round(s_us, 1),
                         "compact_us": round(c_us, 1), "bytes": nbytes,
                         "GBps": round(nbytes / ((s_us + c_us) * 1e-6) / 1e9, 1)})
        del k, v
        torch.cuda.empty_cache()
    return {"workload": "qwen2.5-1.5b-like decode-time eviction sweep (28 layers x 2 KV heads, d=128, fp16)",
            "runs": runs, "caches": "flushed before every run (512 MiB fill, untimed)", "cells": rows,
            "all_cells": {"bound": "hbm", "bytes": tot_bytes, "us": round(tot_us, 1),
                          "achieved": round(tot_bytes / (tot_us * 1e-6) / 1e9, 3), "peak": PEAK_HBM_BYTES / 1e9,
                          "unit": "GB/s", "frac": round(tot_bytes / (tot_us * 1e-6) / PEAK_HBM_BYTES, 4)}}


def under_profiler():
    """True inside a rocprofv3 run. Its preloaded library starts the GPU runtime
    in every child process, so a child that replaces itself with another
    program (the SMI tools are scripts started through /usr/bin/env) must not
    be spawned there."""
    return any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")


def clock_state(keep_busy=None):
    """The GPU's current clocks as the SMI tools report them (None if neither
    runs; not queried under a profiler). `keep_busy`, if given, is called
    (and must wait for its own work) over and over while the query runs, so
    that the tool samples the clocks under that load and not after it."""
    if under_profiler():
        return {"skipped": "not queried under a profiler"}
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            continue
        t_end = time.perf_counter() + 30.0
        busy_calls = 0
        while keep_busy is not None and proc.poll() is None and time.perf_counter() < t_end:
            keep_busy()
            busy_calls += 1
        try:
            out, _ = proc.communicate(timeout=max(1.0, t_end - time.perf_counter()))
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.communicate()
            continue
        if proc.returncode == 0 and out.strip():
            try:
                rep = json.loads(out)
            except ValueError:
                return {"tool": cmd[0], "report": out.strip()[:2000]}
            return {"tool": cmd[0], "clocks_mhz": _clock_values(rep), "steps_run_during_query": busy_calls}
    return None


def _clock_values(rep):
    """{clock name: [current MHz per instance]} from an SMI JSON report."""
    out = {}

    def walk(x, name=None):
        if isinstance(x, dict):
            if "clk" in x and isinstance(x["clk"], dict) and "value" in x["clk"]:
                key = (name or "clk").rstrip("_0123456789")
                out.setdefault(key, []).append(x["clk"]["value"])
                return
            for k, v in x.items():
                walk(v, k)
        elif isinstance(x, list):
            for v in x:
                walk(v, name)
    walk(rep)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def time_step(wl, q, k, v, steps, warmup, stream, flushed_reps=0, clocks=None):
    """Time `steps` steps of the path on one workload (HIP events on the
    launch stream); optionally repeat select + compact after a 512 MiB fill
    that evicts the L2s and the MALL. `clocks`, a list, receives the clock
    state read while the timed steps run."""
    dev = q.device
    bi = wl.budget_inputs()
    budgets = (fam.fam_budgets_from_ratios(bi["ratios"], bi["t"]).tolist() if "ratios" in bi
               else [bi["uniform"]] * wl.Hkv)
    kept, offsets_host = fam.evict_plan(budgets, wl.S, wl.sinks, wl.recent)
    total = int(offsets_host[-1])
    B, Hq, Hkv, S, d = 1, wl.Hq, wl.Hkv, wl.S, wl.d
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
    idx = torch.empty(total, dtype=torch.int32, device=dev)
    offsets = torch.empty(Hkv + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(16, fam.evict_select_workspace_size(Hkv, S, wl.sinks, wl.recent)),
                     dtype=torch.uint8, device=dev)
    k_new = torch.empty((total, d), dtype=k.dtype, device=dev)
    v_new = torch.empty((total, d), dtype=v.dtype, device=dev)
    knorm = torch.empty((B, Hkv, fam.fam_key_norm_parts(S)), dtype=torch.float32, device=dev)
    mass_ws = torch.empty(max(16, fam.fam_mass_workspace_size(B, Hq, Hkv, S)), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]

    def step(events=None):
        if events:
            events[0].record(stream)
        fam.fam_key_norms(k, knorm=knorm)
        fam.fam_lse(q, k, lse=lse, knorm=knorm)
        if events:
            events[1].record(stream)
        # the mass pass's reduction also builds the selection's first
        # histograms (budget-free), so the select that follows starts at
        # its second launch
        fam.fam_mass_prepare_select(q, k, lse, wl.W, wl.sinks, wl.recent, mass=mass, mass_workspace=mass_ws,
                                    select_workspace=ws)
        if events:
            events[2].record(stream)
        fam.evict_select_prepared(mass[0], budgets, wl.sinks, wl.recent, ws, idx=idx, offsets=offsets)
        if events:
            events[3].record(stream)
        fam.kv_compact(k[0], v[0], idx, offsets, total, k_new=k_new, v_new=v_new)
        if events:
            events[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if clocks is not None:   # after the timed steps, under more of the same steps (untimed)
        def busy():
            step()
            torch.cuda.synchronize()
        clocks.append(clock_state(busy))

    names = ["fam_lse", "fam_mass", "evict_select", "kv_compact"]
    per_step = {n: [ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)] for j, n in enumerate(names)}
    ms = {n: float(np.mean(v)) for n, v in per_step.items()}
    work = algorithmic_work(wl, total)
    t_fam = (ms["fam_lse"] + ms["fam_mass"]) * 1e-3
    t_ec = (ms["evict_select"] + ms["kv_compact"]) * 1e-3
    lines = {
        "fam_lse": ("mfma", work["lse_flops"] / (ms["fam_lse"] * 1e-3), PEAK_BF16_FLOPS, "TFLOP/s"),
        "fam_mass": ("mfma", work["mass_flops"] / (ms["fam_mass"] * 1e-3), PEAK_BF16_FLOPS, "TFLOP/s"),
        "evict_select": ("hbm", work["select_bytes"] / (ms["evict_select"] * 1e-3), PEAK_HBM_BYTES, "GB/s"),
        "kv_compact": ("hbm", work["compact_bytes"] / (ms["kv_compact"] * 1e-3), PEAK_HBM_BYTES, "GB/s"),
    }
    flushed = None
    if flushed_reps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fe = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(flushed_reps)]
        for i, e in enumerate(fe):
            flush.fill_(i & 0x7f)
            e[0].record(stream)
            fam.evict_select_prepared(mass[0], budgets, wl.sinks, wl.recent, ws, idx=idx, offsets=offsets)
            e[1].record(stream)
            fam.kv_compact(k[0], v[0], idx, offsets, total, k_new=k_new, v_new=v_new)
            e[2].record(stream)
        torch.cuda.synchronize()
        sel_us = float(np.median([e[0].elapsed_time(e[1]) for e in fe])) * 1e3
        # the whole evict_select (its own histogram launch included), warm and
        # after the fill, for comparison with the prepared form of the step
        full = {}
        for mode in ("warm", "flushed"):
            xe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(flushed_reps)]
            for i, e in enumerate(xe):
                if mode == "flushed":
                    flush.fill_(i & 0x7f)
                e[0].record(stream)
                fam.evict_select(mass[0], budgets, wl.sinks, wl.recent, idx=idx, offsets=offsets, workspace=ws)
                e[1].record(stream)
            torch.cuda.synchronize()
            full[mode] = round(float(np.median([e[0].elapsed_time(e[1]) for e in xe])) * 1e3, 1)
        # the full call rewrote the workspace for the same scores: still prepared
        cmp_us = float(np.median([e[1].elapsed_time(e[2]) for e in fe])) * 1e3
        nbytes = work["select_bytes"] + work["compact_bytes"]
        flushed = {"reps": flushed_reps, "caches": "512 MiB fill before every rep (untimed)",
                   "select_us": round(sel_us, 1), "compact_us": round(cmp_us, 1), "bytes": nbytes,
                   "evict_select_whole_us": full,
                   "GBps": round(nbytes / ((sel_us + cmp_us) * 1e-6) / 1e9, 1),
                   "hbm_frac": round(nbytes / ((sel_us + cmp_us) * 1e-6) / PEAK_HBM_BYTES, 4)}
        # what a plain device copy of the compaction's bytes (the kept K and V
        # rows read once and written once) reaches on this machine, warm and
        # after the same fill: the practical ceiling of the HBM-bound kernels
        half = work["compact_bytes"] // 2
        src = torch.empty(half, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ref = {}
        for mode in ("warm", "flushed"):
            ce = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(flushed_reps)]
            dst.copy_(src)
            for i, e in enumerate(ce):
                if mode == "flushed":
                    flush.fill_(i & 0x7f)
                e[0].record(stream)
                dst.copy_(src)
                e[1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([e[0].elapsed_time(e[1]) for e in ce])) * 1e3
            ref[mode] = {"us": round(us, 1), "GBps": round(2 * half / (us * 1e-6) / 1e9, 1)}
        flushed["copy_reference"] = dict(ref, bytes=2 * half, kernel="torch copy_ (device to device)")
        del flush, src, dst
    return {"names": names, "ms": ms, "per_step": per_step, "lines": lines, "work": work,
            "budgets": budgets, "total": total, "mass": mass, "lse": lse, "idx": idx, "offsets": offsets,
            "ms_step": wall * 1e3 / steps, "t_fam": t_fam, "t_ec": t_ec, "flushed": flushed}


def mass_select_row(reps, q, k, wl, run, stream, derive=False):
    """fam_mass_select against fam_mass followed by evict_select on the same
    workload (HIP events on the launch stream, the forms alternating in every
    rep). At 128k both forms spend about 57 ms in the mass pass, whose
    run-to-run spread is far larger than the launch the combined form saves,
    so only the totals are reported there and the saving is read from a kernel
    trace (end of the mass pass to the end of the last select launch). With
    `derive` (short workloads, whose mass pass is short enough), fam_mass and
    evict_select are timed apart too, and the selection's share of the
    combined call (its time minus fam_mass's, paired per rep) gives the
    select + compact rate of the combined form."""
    dev = q.device
    B, Hq, Hkv, S = 1, wl.Hq, wl.Hkv, wl.S
    lse, budgets, total, work = run["lse"], run["budgets"], run["total"], run["work"]
    mass = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
    idx = torch.empty(total, dtype=torch.int32, device=dev)
    offsets = torch.empty(Hkv + 1, dtype=torch.int64, device=dev)
    mws = torch.empty(max(16, fam.fam_mass_workspace_size(B, Hq, Hkv, S)), dtype=torch.uint8, device=dev)
    sws = torch.empty(max(16, fam.evict_select_workspace_size(Hkv, S, wl.sinks, wl.recent)),
                      dtype=torch.uint8, device=dev)

    def fused():
        fam.fam_mass_select(q, k, lse, wl.W, budgets, wl.sinks, wl.recent, mass=mass, idx=idx,
                            offsets=offsets, mass_workspace=mws, select_workspace=sws)

    def mass_only():
        fam.fam_mass(q, k, lse, wl.W, mass=mass, workspace=mws)

    def select_only():
        fam.evict_select(mass[0], budgets, wl.sinks, wl.recent, idx=idx, offsets=offsets, workspace=sws)

    fused()
    mass_only()
    select_only()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        fused()
        e[1].record(stream)
        mass_only()
        if derive:
            e[2].record(stream)
        select_only()
        e[3].record(stream)
    torch.cuda.synchronize()
    f = [e[0].elapsed_time(e[1]) for e in ev]
    a = [e[1].elapsed_time(e[3]) for e in ev]
    out = {"reps": reps, "ms_median": {"fam_mass_select": round(float(np.median(f)), 4),
                                       "fam_mass + evict_select": round(float(np.median(a)), 4)},
           "ms_spread": {"fam_mass_select": round(max(f) - min(f), 4),
                         "fam_mass + evict_select": round(max(a) - min(a), 4)}}
    if derive:
        m = [e[1].elapsed_time(e[2]) for e in ev]
        sel = [e[2].elapsed_time(e[3]) for e in ev]
        share = float(np.median([fi - mi for fi, mi in zip(f, m)])) * 1e3
        nbytes = work["select_bytes"] + work["compact_bytes"]
        rate = nbytes / ((share + run["ms"]["kv_compact"] * 1e3) * 1e-6)
        out.update({"fam_mass_ms_median": round(float(np.median(m)), 4),
                    "evict_select_us_median": round(float(np.median(sel)) * 1e3, 1),
                    "select_us_in_fam_mass_select": round(share, 1),
                    "evict_compact_gbps_combined": round(rate / 1e9, 2),
                    "evict_compact_hbm_frac_combined": round(rate / PEAK_HBM_BYTES, 4)})
    return out


def workload_row(wl, steps, warmup, stream, mass_select_reps=0, oracle_select=False):
    """One more workload's step, timed on its own inputs (for the lines of
    the other score workloads beside the headline one); with `oracle_select`,
    the oracle's select + compact on the same masses and K/V, timed on the
    host."""
    dev = torch.device("cuda:0")
    t = wl.tensors()
    q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
    del t
    run = time_step(wl, q, k, v, steps, warmup, stream)
    ms, work = run["ms"], run["work"]
    out = {"workload": wl.name, "steps": steps,
           "config": {"q_heads": wl.Hq, "kv_heads": wl.Hkv, "seq_len": wl.S, "head_dim": wl.d, "window": wl.W,
                      "sinks": wl.sinks, "kept_total": run["total"]},
           "pairs_per_s": work["causal_pairs"] / (run["ms_step"] * 1e-3),
           "fam_mfma_frac": round((work["lse_flops"] + work["mass_flops"]) / run["t_fam"] / PEAK_BF16_FLOPS, 4),
           "evict_compact_gbps": round((work["select_bytes"] + work["compact_bytes"]) / run["t_ec"] / 1e9, 2),
           "evict_compact_hbm_frac": round((work["select_bytes"] + work["compact_bytes"]) / run["t_ec"]
                                           / PEAK_HBM_BYTES, 4),
           "kernel_ms": {n: round(ms[n], 4) for n in run["names"]}}
    if mass_select_reps > 0:
        out["mass_select"] = mass_select_row(mass_select_reps, q, k, wl, run, stream, derive=True)
    if oracle_select:
        host = {"mass": run["mass"][0].cpu().numpy(), "k": k[0].cpu().view(torch.int16).numpy(),
                "v": v[0].cpu().view(torch.int16).numpy(), "budgets": run["budgets"]}
        out["cpu_oracle_select_compact"] = oracle_select_compact(wl, host, False)[wl.name]
    del q, k, v, run
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama-128k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--target-steps", type=int, default=2,
                    help="timed runs of the KVpop target row (per-head mass + epilogue); 0 skips it")
    ap.add_argument("--chunked-runs", type=int, default=1,
                    help="timed runs of the chunked prefill-compress loop; 0 skips it")
    ap.add_argument("--ranking-runs", type=int, default=3,
                    help="timed runs of the ranking-quality row; 0 skips it")
    ap.add_argument("--decode-runs", type=int, default=5,
                    help="timed runs per cell of the decode-time eviction sweep; 0 skips it")
    ap.add_argument("--chunked-only", action="store_true",
                    help="run only the chunked prefill-compress row (for a kernel trace of it alone)")
    ap.add_argument("--other-workloads", type=int, default=5,
                    help="timed steps of the 8k and 32k score workloads beside the 128k line; 0 skips them")
    ap.add_argument("--flushed-reps", type=int, default=5,
                    help="select + compact reps after a cache-evicting fill (headline workload); 0 skips them")
    ap.add_argument("--mass-select-reps", type=int, default=5,
                    help="reps of fam_mass_select against fam_mass + evict_select (headline workload); 0 skips them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no exchange, so one GPU shows its full per-GPU shape)", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    wl = WORKLOADS[args.workload]()
    t = wl.tensors()
    q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
    del t
    stream = torch.cuda.current_stream(dev)
    if args.chunked_only:
        print(json.dumps({"chunked_prefill": chunked_row(max(1, args.chunked_runs), q, k, v, wl, stream)}),
              flush=True)
        return
    clocks = []
    run = time_step(wl, q, k, v, args.steps, args.warmup, stream, flushed_reps=args.flushed_reps, clocks=clocks)
    names, ms, per_step, lines, work = run["names"], run["ms"], run["per_step"], run["lines"], run["work"]
    budgets, total, mass, lse = run["budgets"], run["total"], run["mass"], run["lse"]
    B, Hq, Hkv, S = 1, wl.Hq, wl.Hkv, wl.S
    ms_step = run["ms_step"]
    t_fam, t_ec = run["t_fam"], run["t_ec"]
    traffic = measured_traffic(args.workload)
    roof = {}
    for n, (bound, ach, peak, unit) in lines.items():
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        roof[n] = {"bound": bound, "achieved": round(ach / scale, 3), "peak": peak / scale,
                   "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic.get(n),
                   "ms": round(ms[n], 4)}
    dominant = max(names, key=lambda n: ms[n])
    out = {
        "metric": "future-attn-mass causal key-query pairs/s (+ % bf16 MFMA peak; evict+compact GB/s)",
        "value": work["causal_pairs"] / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "q_heads": Hq, "kv_heads": Hkv, "seq_len": S,
                   "head_dim": wl.d, "window": wl.W, "sinks": wl.sinks, "recent": wl.recent,
                   "kept_total": total, "budgets": [int(b) for b in budgets]},
        "step_calls": ["fam_key_norms", "fam_lse", "fam_mass_prepare_select", "evict_select_prepared",
                       "kv_compact"],
        "fam_mfma_frac": round((work["lse_flops"] + work["mass_flops"]) / t_fam / PEAK_BF16_FLOPS, 4),
        "fam_pairs_per_s": work["causal_pairs"] / t_fam,
        "evict_compact_gbps": round((work["select_bytes"] + work["compact_bytes"]) / t_ec / 1e9, 2),
        "evict_compact_hbm_frac": round((work["select_bytes"] + work["compact_bytes"]) / t_ec / PEAK_HBM_BYTES, 4),
        "kernel_ms": {n: round(ms[n], 4) for n in names},
        "kernel_ms_median": {n: round(float(np.median(per_step[n])), 4) for n in names},
        "kernel_ms_min": {n: round(float(np.min(per_step[n])), 4) for n in names},
        "roofline": dict(roof[dominant], kernel=dominant),
        "roofline_all": roof,
        "evict_compact_flushed": run["flushed"],
        "clock_state_during_steps": clocks[0] if clocks else None,
    }
    if args.mass_select_reps > 0:
        out["mass_select"] = mass_select_row(args.mass_select_reps, q, k, wl, run, stream)
    if args.target_steps > 0:
        out["kvpop_target"] = kvpop_target_row(args.target_steps, q, k, lse, wl, work, stream)
        for n in ("fam_mass_per_head", "fam_kvpop_target"):
            out["kvpop_target"][n]["traffic"] = traffic.get(n)
    if args.ranking_runs > 0:
        out["ranking"] = ranking_row(args.ranking_runs, mass, wl, stream)
    if args.chunked_runs > 0:
        out["chunked_prefill"] = chunked_row(args.chunked_runs, q, k, v, wl, stream)
    if args.decode_runs > 0:
        out["decode_sweep"] = decode_row(args.decode_runs, stream)
    host = None
    if not args.no_cpu_baseline:   # host copies for the oracle's select + compact, taken before freeing
        host = {"mass": mass[0].cpu().numpy(), "k": k[0].cpu().view(torch.int16).numpy(),
                "v": v[0].cpu().view(torch.int16).numpy(), "budgets": budgets}
    del q, k, v, mass, lse, run
    torch.cuda.empty_cache()
    if args.other_workloads > 0 and args.workload == "llama-128k":
        out["other_workloads"] = [workload_row(WORKLOADS[n](), args.other_workloads, 1, stream,
                                               4 * args.mass_select_reps, not args.no_cpu_baseline)
                                  for n in ("qwen3-4b-8k", "long-trace-32k")]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
        out["cpu_baseline"]["cpu_model"] = cpu_model()
        out["cpu_baseline"]["select_compact"] = oracle_select_compact(wl, host, args.decode_runs > 0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
