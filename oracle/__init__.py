"""CPU oracle for one CSA2 compressed-sparse-attention layer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or execute anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code, table or helper with the GPU path.

Everything here is plain numpy in float64 (the method's own precision choices,
such as "round to fp32 before quantizing", are applied explicitly where the
method makes them).  Each function cites the passage it follows.

Sources
-------
"DeepSeek-V4.1 架构解析：把长上下文的成本瓶颈从算力挪到存储"
    (blog.yuzhonghai.cloud/deepseek-v41-arch), sections
    "02 CSA2：大多数层不再自己算注意力" (layer modes, Top-512, the 2,048-block x 8
    hierarchical pool) and "03 精度与状态重建" (MXFP4 = E2M1 values with one E4M3
    scale per 16 channels, no global scale, 448 x 6 = 2688 range, quantize after
    RoPE, FP4 for storage only, SWA KV in FP8, n_win = 128); cited in the
    docstrings as "DeepSeek-V4.1 架构解析" §NN.
The DeepSeek V4 overview page (wmrh.cn/news/159405), section 2.1 (4:1 sequence
    compression of the CSA predecessor).

Readings where the pages are silent (the pages give no formula for the
compressor or the indexer and no dimensions) are stated in each function's
docstring and collected in the repository's design notes.

Parity status
-------------
Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself (library routines, closed forms, page constants, brute force on
tiny inputs) except the RoPE *conventions* (which channels, pairing, base,
position): the pages say only "quantize after RoPE" and "RoPE preserves the
norm", so those conventions are parity unpinned; the rotation itself is pinned.
"""

from .formats import (
    E2M1_VALUES,
    e4m3_decode,
    e4m3_encode,
    e2m1_decode,
    e2m1_encode,
)
from .mxfp4 import quantize, dequantize, GROUP
from .compressor import compress, rope_rotate, compress_rope_fp32
from .indexer import visible_entries, index_scores, index_scores_many, pooled_entries
from .select import topk, block_pool
from .attention import window_positions, sparse_attention
from .layer import LayerState, layer_full, layer_reindex, layer_reuse, window_encode, window_rebuild

__all__ = [
    "E2M1_VALUES", "e4m3_decode", "e4m3_encode", "e2m1_decode", "e2m1_encode",
    "quantize", "dequantize", "GROUP",
    "compress", "rope_rotate", "compress_rope_fp32",
    "visible_entries", "index_scores", "index_scores_many", "pooled_entries",
    "topk", "block_pool",
    "window_positions", "sparse_attention",
    "LayerState", "layer_full", "layer_reindex", "layer_reuse", "window_encode", "window_rebuild",
]
