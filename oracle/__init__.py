"""CPU oracle for exact attention: test infrastructure only.

Plain, slow, fp64 numpy definitions of what the attention path computes.
Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from here.  The product path (the HIP
library and its Python binding) never imports, calls or links this package,
and this package never imports the product path: the two share no code.

Sources (web pages) cited in this package:
  [TA]  "Accelerating AI: A Deep Dive into Flash Attention and Its Impacts"
        (Towards AI article)
  [FA]  "FlashAttention: Fast and Memory-Efficient Exact Attention"
        (repository overview of Dao-AILab/flash-attention)
  [HF]  "Improvements in attention_forward functions"
        (huggingface/transformers issue 36218)
  [GYM] "FlexAttention uses much more GPU memory than FlashAttention-2"
        (pytorch-labs/attention-gym issue 101)
  [FX4] "Lightning Talk: FlexAttention + FlashAttention-4: Fast and Flexible"
        (PyTorch Conference Europe 2026)

Every function here is pinned by a CPU test against something other than
itself (closed forms, library routines, brute-force loops, finite
differences).  No function is parity-unpinned.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    allowed_pair_count,
    attention_bwd,
    attention_fwd,
    attention_fwd_rows,
    block_mask,
    combine_partials,
    decode,
    decode_split,
    kv_head_of,
)
from .kvcache import cache_rows, decode_kvcache, kvcache_append  # noqa: F401
