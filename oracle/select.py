"""Top-K selection and the hierarchical block pool.

"DeepSeek-V4.1 架构解析" §02: the first Full layer of the decoder scans every visible position and
picks the Top-512; it then ranks blocks of 8 positions by the largest index
score inside each block and keeps 2,048 blocks, a shared pool of 16,384
candidates in which the following Reindex layers search.

Readings where the page is silent:
  * equal scores are ordered by the lower entry index (and equal block maxima
    by the lower block index); the two rules must agree for the pool to contain
    the Top-K (see the tests of this module);
  * the selected ids are returned in ascending order, padded with -1 when fewer
    than K entries are visible;
  * blocks are aligned runs of 8 consecutive entries; a partially visible last
    block uses its visible entries only; with at most 2,048 blocks the pool is
    every visible entry.
"""

import numpy as np


def topk(scores, k, ids=None):
    """The k best (score desc, id asc) of ``scores``; ascending ids, -1 padded.

    scores: float64 [N]; ids: the entry id of each score (default 0..N-1).
    """
    scores = np.asarray(scores, dtype=np.float64)
    ids = np.arange(len(scores)) if ids is None else np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -scores))   # primary: -score, secondary: id
    chosen = np.sort(ids[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


def block_max(scores, block=8):
    """Max over aligned blocks of ``block`` consecutive entries (last may be partial)."""
    scores = np.asarray(scores, dtype=np.float64)
    nb = (len(scores) + block - 1) // block
    padded = np.full(nb * block, -np.inf)      # the missing tail of a partial block adds nothing
    padded[:len(scores)] = scores
    return padded.reshape(nb, block).max(axis=1)


def block_pool(scores, n_blocks=2048, block=8):
    """Ids of the n_blocks blocks with the largest block max; ascending, -1 padded.

    ``scores`` are the scores of the visible prefix (entries 0..nv-1).
    """
    bm = block_max(scores, block)
    return topk(bm, n_blocks)
