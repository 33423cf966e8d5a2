"""Indexer scoring over the causally visible entries.

"DeepSeek-V4.1 架构解析" §02: a Full-mode layer computes its own indexer K and scores every causally
visible position to pick the Top-512; a Reindex layer reuses the previous
layer's global KV and indexer K but scores with its own indexer query; with the
hierarchical pool, Reindex layers score only inside the 16,384-entry pool.

Readings where the page is silent (it gives no scoring formula):
  * score_j = sum_h w_h * ReLU(q_h . k_j) with 8 indexer heads of 128 dims,
    q and k stored as E4M3 bytes and w float32 per query and head;
  * entry j is visible to a query at token position p iff its last token is not
    after p: 4j + 3 <= p, i.e. the visible set is the prefix j < (p + 1) // 4.

In float64 the dot products are exact in any order: every E4M3 value is an
integer multiple of 2**-9 with magnitude <= 448, so each product is a multiple
of 2**-18 below 2**18 and a 128-term sum needs fewer than 44 significant bits.
"""

import numpy as np

from .formats import e4m3_decode


def visible_entries(q_pos, n_entries=None):
    """Number of entries visible at token position p: (p + 1) // 4."""
    nv = (int(q_pos) + 1) // 4
    if n_entries is not None:
        nv = min(nv, int(n_entries))
    return nv


def index_scores(q_fp8, w, k_fp8, entries=None, k_values=None):
    """Scores of one query against a set of indexer keys.

    q_fp8: [H_I, d_I] E4M3 bytes; w: [H_I] float32; k_fp8: [N, d_I] E4M3 bytes.
    ``entries`` (optional) selects rows of k_fp8 (the pooled case).
    ``k_values`` (optional): the keys already decoded to float64, [N, d_I]
    (the same rows as k_fp8; used instead of decoding k_fp8 again).
    Returns float64 [len(entries) or N].
    """
    q = e4m3_decode(q_fp8)
    if k_values is None:
        k = e4m3_decode(k_fp8 if entries is None else np.asarray(k_fp8)[np.asarray(entries)])
    else:
        k = k_values if entries is None else np.asarray(k_values)[np.asarray(entries)]
    dots = k @ q.T                       # [N, H_I], exact
    relu = np.maximum(dots, 0.0)
    return relu @ np.asarray(w, dtype=np.float64)


def index_scores_many(q_fp8, w, k_values):
    """Scores of several queries against the same decoded keys (the prefill
    case, where a chunk's queries share the sequence's keys).

    q_fp8: [nq, H_I, d_I] E4M3 bytes; w: [nq, H_I] float32; k_values:
    [N, d_I] float64 decoded keys.  Returns float64 [nq, N]; row i is
    index_scores(q_fp8[i], w[i], keys) up to the order of the final 8-term
    weighted sum.
    """
    q = e4m3_decode(q_fp8)
    nq, h, d = q.shape
    dots = (q.reshape(nq * h, d) @ np.asarray(k_values).T).reshape(nq, h, -1)   # exact
    relu = np.maximum(dots, 0.0)
    return np.matmul(np.asarray(w, dtype=np.float64)[:, None, :], relu)[:, 0, :]


def pooled_entries(pool_blocks, n_visible, block=8):
    """Visible entries of the pool blocks, ascending (block ids ascending).

    Pool block b holds entries block*b .. block*b + block - 1; -1 slots are
    empty; entries at or past n_visible (the tail of a partly visible last
    block, or blocks past the visible prefix) are not candidates.
    """
    b = np.asarray(pool_blocks, dtype=np.int64).reshape(-1)
    b = b[b >= 0]
    ids = (block * b[:, None] + np.arange(block, dtype=np.int64)[None, :]).reshape(-1)
    return np.sort(ids[ids < int(n_visible)])
