"""Sparse multi-query attention over selected entries plus the FP8 window.

"DeepSeek-V4.1 架构解析" §02: the selected Top-K entries are "taken to do attention"; CSA2 shrinks the
number of KV heads (one shared latent serves all query heads).  "DeepSeek-V4.1 架构解析" §03: the
FP4 cache is dequantized before attention, the sliding-window (SWA) KV stays in
FP8, and the window is n_win = 128 tokens.

Readings where the pages are silent:
  * multi-query attention with one 512-d latent used as both key and value,
    16 query heads, logits scaled by 1/sqrt(512);
  * the key set of a query at position p is the union of the dequantized
    selected entries and the window tokens max(0, p-127) .. p (E4M3 bytes
    decoded without a scale), under one softmax normalizer; an entry and a
    window token that cover the same positions are both kept.
"""

import numpy as np

from .formats import e4m3_decode
from .mxfp4 import dequantize

N_WIN = 128


def window_positions(p, n_win=N_WIN):
    """Token positions of the sliding window of a query at position p."""
    return np.arange(max(0, int(p) - n_win + 1), int(p) + 1)


def sparse_attention(q, codes, scales, idx, win_fp8, sm_scale):
    """One query's attention output [H, D] in float64.

    q: [H, D] float32; codes [N, D/2] / scales [N, D/16]: the entry cache;
    idx: selected entry ids (-1 entries are skipped); win_fp8: [W, D] E4M3
    bytes of the window tokens in position order.
    """
    q = np.asarray(q, dtype=np.float64)
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    keys = [dequantize(np.asarray(codes)[idx], np.asarray(scales)[idx])]
    keys.append(e4m3_decode(np.asarray(win_fp8)))
    kv = np.concatenate(keys, axis=0)            # [n_keys, D]; K = V
    logits = (q @ kv.T) * float(sm_scale)        # [H, n_keys]
    m = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ kv
