"""The three CSA2 layer modes and window maintenance, one query at a time.

"DeepSeek-V4.1 架构解析" §02: each layer has a statically assigned mode.
  Full     computes its own main KV, indexer K and Top-K indices;
  Reindex  reuses the previous layer's global KV and indexer K, rescoring with
           its own indexer query to pick a new Top-K (only inside the
           hierarchical pool when one was built);
  Reuse    keeps the most recent Top-K indices and only runs attention.
"DeepSeek-V4.1 架构解析" §02 also says the first Full layer builds the pool from its own scores.
"DeepSeek-V4.1 架构解析" §03: the SWA KV is kept in FP8 and bounded to n_win = 128 tokens.

Reading where the page is silent: a Reuse layer uses the indices of the most
recent Full or Reindex layer before it; window tokens are the raw token
latents rounded to E4M3 (RNE, saturating, no scale).
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .attention import sparse_attention
from .formats import e4m3_encode
from .indexer import index_scores, pooled_entries, visible_entries
from .select import block_pool, topk

TOP_K = 512
POOL_BLOCKS = 2048
BLOCK = 8


@dataclass
class LayerState:
    """Per-query outputs of a layer."""
    idx: np.ndarray
    out: np.ndarray
    pool: Optional[np.ndarray] = None
    scores: Optional[np.ndarray] = None


def window_encode(x_tokens):
    """Window maintenance: token latents (float32) -> E4M3 bytes."""
    return e4m3_encode(np.asarray(x_tokens, dtype=np.float32))


def window_rebuild(x_last, p_last, win_cap):
    """SWA Bounded Replay ("DeepSeek-V4.1 架构解析" §03): the window ring rebuilt from the latest
    tokens only.  x_last float32 [n_tok, 512] are the tokens at positions
    p_last - n_tok + 1 .. p_last (n_tok <= win_cap); the token at position t
    goes to row t % win_cap, rows no given token reaches stay zero.  Returns
    uint8 [win_cap, 512]."""
    x_last = np.asarray(x_last, dtype=np.float32)
    n_tok = x_last.shape[0]
    assert 1 <= n_tok <= win_cap
    ring = np.zeros((win_cap, x_last.shape[1]), dtype=np.uint8)
    for i in range(n_tok):
        t = p_last - (n_tok - 1 - i)
        if t >= 0:
            ring[t % win_cap] = window_encode(x_last[i])
    return ring


def layer_full(codes, scales, k_fp8, q_fp8, w, q_attn, q_pos, win_fp8, sm_scale,
               build_pool=False, k=TOP_K, n_blocks=POOL_BLOCKS, n_entries=None,
               k_values=None, scores=None, attend=True):
    """Full mode for one query: score all visible entries, Top-K, attention.

    k_values: optional float64 decoded keys (rows of k_fp8); scores: optional
    scores of the visible entries computed beforehand (index_scores_many);
    attend=False skips the attention (out is None).
    """
    nv = visible_entries(q_pos, n_entries if n_entries is not None else len(k_fp8))
    if scores is None:
        scores = index_scores(q_fp8, w, np.asarray(k_fp8)[:nv],
                              k_values=None if k_values is None else np.asarray(k_values)[:nv])
    idx = topk(scores, k)
    pool = block_pool(scores, n_blocks, BLOCK) if build_pool else None
    out = sparse_attention(q_attn, codes, scales, idx, win_fp8, sm_scale) if attend else None
    return LayerState(idx=idx, out=out, pool=pool, scores=scores)


def layer_reindex(codes, scales, k_fp8, pool, q_fp8, w, q_attn, q_pos, win_fp8,
                  sm_scale, k=TOP_K, n_entries=None, k_values=None, attend=True):
    """Reindex mode: rescore with this layer's query, inside the pool if given."""
    nv = visible_entries(q_pos, n_entries if n_entries is not None else len(k_fp8))
    if pool is None:
        ids = np.arange(nv)
    else:
        ids = pooled_entries(pool, nv, BLOCK)
    scores = index_scores(q_fp8, w, k_fp8, entries=ids, k_values=k_values)
    idx = topk(scores, k, ids=ids)
    out = sparse_attention(q_attn, codes, scales, idx, win_fp8, sm_scale) if attend else None
    return LayerState(idx=idx, out=out, pool=pool, scores=scores)


def layer_reuse(codes, scales, idx, q_attn, win_fp8, sm_scale, attend=True):
    """Reuse mode: attention with the most recent Top-K indices."""
    out = sparse_attention(q_attn, codes, scales, idx, win_fp8, sm_scale) if attend else None
    return LayerState(idx=np.asarray(idx), out=out)
