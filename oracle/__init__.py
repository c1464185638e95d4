"""Plain fp64 CPU oracle for future-attention mass and budgeted eviction.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it. It shares no code, tables or
helpers with the HIP library and imports nothing from it.

Modules
  fam_oracle      causal row log-sum-exp and future-attention mass
  select_oracle   budget plan, sort-based top-k selection, compaction
  soft_topk       closed-form Soft-TopK and per-head budgets (LKV)
  kvpop_target    count-normalised log target and group aggregation (KVpop)
  chunked         chunked prefill with compression after every chunk (KVP)
  ranking         eviction cost over budgets and retention recall (KVP, KVpop)
  topk_cutoff     running top-k cut-off over static ranks (KVpop)

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``
against brute force, closed forms, invariants or the pages' worked example.
"""
from . import chunked, fam_oracle, kvpop_target, ranking, select_oracle, soft_topk, topk_cutoff  # noqa: F401
