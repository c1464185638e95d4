"""Write the full-size fp64 oracle fixtures of the 32k and 128k workloads.

Run from the repository root: ``python tests/golden/make_fullsize_goldens.py``
(minutes on a few cores). It calls only ``oracle/`` and the seeded input
generators of ``future_attention_scoring_amd.workloads`` (which hold none of
the method's arithmetic), and writes:

* ``long_trace_s32768_group0.npz``: the long reasoning trace (32 query / 8
  KV heads, d=128, S=32768, W=256, mixture keys), KV group 0: the causal LSE
  of its 4 query heads at every row and the group's future mass at every key.
* ``llama_s131072_group0.npz``: the Llama-3.1-8B-like layer (32 / 8 heads,
  d=128, S=131072, W=512), KV group 0: the causal LSE of its 4 query heads at
  every row and the group's future mass at 288 keys spread over the whole
  sequence (the sinks, early keys, an even spread, the window edge and the
  first unreachable keys).

Both hold the SHA-256 of the bf16 input bytes they were computed from, so a
change of the generators shows up as a hash mismatch rather than as a parity
failure. The query heads' normalisers are computed one head per process
(each a call of the oracle's causal LSE on that head alone); the masses are
one oracle call over the whole group.
"""
from __future__ import annotations

import hashlib
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

HERE = os.path.dirname(os.path.abspath(__file__))


def group_inputs(wl, group):
    """bf16-rounded Q of the group's query heads and K of its KV head, as fp64."""
    import torch
    g = wl.group
    t = wl.tensors(q_heads=range(group * g, (group + 1) * g), kv_heads=[group], with_v=False)
    q16, k16 = t["q"][0], t["k"][0, 0]
    sha = hashlib.sha256(q16.view(torch.int16).numpy().tobytes() + k16.view(torch.int16).numpy().tobytes())
    return q16.to(torch.float64).numpy(), k16.to(torch.float64).numpy(), sha.hexdigest()


def _lse_one_head(args):
    name, group, n = args
    from future_attention_scoring_amd import workloads
    from oracle import fam_oracle as fo
    wl = getattr(workloads, name)()
    q, k, _ = group_inputs(wl, group)
    t0 = time.time()
    lse = fo.causal_lse(q[n:n + 1], k[None], 1.0 / math.sqrt(wl.d))[0]
    print(f"  {name} head {n}: lse in {time.time() - t0:.0f} s", flush=True)
    return lse


def head_lses(name, group, g, procs):
    with mp.get_context("spawn").Pool(procs) as pool:
        return np.stack(pool.map(_lse_one_head, [(name, group, n) for n in range(g)]))


def llama_keys(S, W):
    """Sinks and early keys, an even spread, the window edge, the first unreachable keys."""
    last = S - W - 1                                   # the last key any query reaches
    early = np.arange(0, 16)
    spread = np.linspace(16, last - 16, 240).round().astype(np.int64)
    edge = np.arange(last - 15, last + 1)
    beyond = np.array([last + 1, last + 2, S - 1])
    return np.unique(np.concatenate([early, spread, edge, beyond]))


def main():
    from future_attention_scoring_amd import workloads
    from oracle import fam_oracle as fo
    procs = int(os.environ.get("GOLDEN_PROCS", "4"))
    os.environ.setdefault("OMP_NUM_THREADS", "2")

    wl = workloads.long_trace()
    q, k, sha = group_inputs(wl, 0)
    t0 = time.time()
    lse = head_lses("long_trace", 0, wl.group, procs)
    mass = fo.future_mass(q, k[None], lse, wl.W, 1.0 / math.sqrt(wl.d))[0]
    print(f"{wl.name}: group 0 in {time.time() - t0:.0f} s", flush=True)
    np.savez(os.path.join(HERE, "long_trace_s32768_group0.npz"), lse=lse, mass=mass,
             S=wl.S, W=wl.W, d=wl.d, group=0, seed=wl.seed, input_sha256=sha)

    wl = workloads.llama31_8b_128k()
    q, k, sha = group_inputs(wl, 0)
    t0 = time.time()
    lse = head_lses("llama31_8b_128k", 0, wl.group, procs)
    keys = llama_keys(wl.S, wl.W)
    mass = fo.future_mass_keys(q, k, lse, 0, keys, wl.W, 1.0 / math.sqrt(wl.d))
    print(f"{wl.name}: group 0 in {time.time() - t0:.0f} s", flush=True)
    np.savez(os.path.join(HERE, "llama_s131072_group0.npz"), lse=lse.astype(np.float32),
             keys=keys, mass=mass, S=wl.S, W=wl.W, d=wl.d, group=0, seed=wl.seed,
             input_sha256=sha)


if __name__ == "__main__":
    main()
