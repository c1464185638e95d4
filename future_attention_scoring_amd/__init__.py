"""Future-attention mass and budgeted KV-cache eviction on MI355X (gfx950).

The compute path is libfam.so (HIP kernels behind a C ABI, see include/fam.h);
``future_attention_scoring_amd.fam`` is its ctypes binding and
``future_attention_scoring_amd.workloads`` draws seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use.
"""

__all__ = ["fam", "workloads"]
