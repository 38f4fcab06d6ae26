"""Per-head heterogeneous block-sparse attention for AMD MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libsparse_attn.so``, built from ``csrc/``); ``sparse_attn`` is its thin
ctypes binding.  ``workloads`` draws the seeded synthetic inputs.  Importing the
package itself loads nothing; ``sparse_attn`` fails loudly if the library is
missing.
"""

__all__ = ["sparse_attn", "workloads"]
