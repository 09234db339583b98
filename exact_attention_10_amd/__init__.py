"""Exact IO-aware tiled attention for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/attn.h`` at the repository root); the
``binding`` module is a thin ctypes layer over it that takes torch tensors
only as device memory and streams.  Importing this package does not load the
library; importing ``exact_attention_10_amd.binding`` does, and fails loudly
when it has not been built.
"""

__all__ = ["binding", "inputs"]
