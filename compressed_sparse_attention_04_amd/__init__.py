"""MI355X-native CSA2 compressed sparse attention layer step.

The computation lives in libcsa.so (hand-written HIP for gfx950, C ABI in
include/csa.h); this package is its Python binding (``ops``), its build
script (``build``) and the layer-step driver used by the benchmark
(``step``).
"""

from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    CsaError,
    csa_quantize,
    csa_dequantize,
    csa_compress_quant,
    csa_window_append,
    csa_index_score,
    csa_topk,
    csa_block_pool,
    csa_sparse_attn,
    csa_layer_full,
    csa_layer_reindex,
    csa_layer_reuse,
    LayerCall,
)
